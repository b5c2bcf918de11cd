// Device workspaces the library keeps per (device, stream, use): the GEMMs'
// split-K partial sums and the decode attention's partial softmax states.
//
// A call that needs a larger buffer than its stream has gets a new one from
// hipMallocAsync on that stream: the allocation is stream-ordered, so the
// call neither waits for work already queued nor synchronises the device.
// The buffer it replaces is retired, not freed: kernels queued earlier, and
// HIP graphs captured earlier on the stream, may still reference it, so it is
// kept until the process ends.  Sizes grow at least twofold, which bounds
// the retired memory by the size of the live buffer.  Growing while the
// stream is being captured into a graph is refused (the allocation would
// become a node of the graph): such a call returns an error instead.
#include "dmq_common.h"

#include <mutex>
#include <vector>

namespace dmq {

namespace {

struct Workspace {
  int dev;
  int use;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};

std::mutex g_ws_mu;
std::vector<Workspace> g_live;
std::vector<void*> g_retired;

constexpr size_t kGranule = size_t(2) << 20;

}  // namespace

hipError_t stream_workspace(WorkspaceUse use, hipStream_t s, size_t bytes, void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  Workspace* w = nullptr;
  for (auto& e : g_live)
    if (e.dev == dev && e.use == (int)use && e.stream == s) w = &e;
  if (w && w->bytes >= bytes) {
    *out = w->ptr;
    return hipSuccess;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if ((err = hipStreamIsCapturing(s, &cs)) != hipSuccess) return err;
  if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
  size_t want = bytes;
  if (w && want < 2 * w->bytes) want = 2 * w->bytes;
  want = (want + kGranule - 1) / kGranule * kGranule;
  void* p = nullptr;
  if ((err = hipMallocAsync(&p, want, s)) != hipSuccess) return err;
  if (w) {
    g_retired.push_back(w->ptr);
    w->ptr = p;
    w->bytes = want;
  } else {
    g_live.push_back(Workspace{dev, (int)use, s, p, want});
  }
  *out = p;
  return hipSuccess;
}

}  // namespace dmq
