// moss_attention_noalloc: the standalone exact attention (moss_attention) without any device
// allocation, for callers that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// moss_attention allocates, per call, the scratch that holds the partial results of the key-split tail
// tiles (when the query tiles leave the chip's last round of workgroups partly empty), and once per
// process the RoPE table. Here both live in file-scope device arrays: `scratch` holds the partial
// results (sized for the largest split any plan makes on a chip of up to 256 compute units: at most
// two workgroups per compute unit take part, 128 queries each, 128 fp32 values plus a (max, sum) pair
// per query), and `rope_static` the RoPE table (theta 1e4). Each GPU holds its own copy of both until
// the process ends. Their device addresses are taken once per device with hipGetSymbolAddress (the
// host-side names are only stand-ins) and used for every launch.
#include <mutex>

#include "kernels.h"
#include "moss_dit_ops.h"

namespace moss {
namespace {

constexpr size_t kScratchBytes = (size_t)MOSS_ATTENTION_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes >= 512UL * kAttnBQ * (kHeadDim + 2) * 4 + 256,
              "the scratch must hold the largest split of a 256-CU chip");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static __device__ __align__(256) float rope_static[kRopeTableFloats];

struct DeviceScratch {
  bool ready = false;
  void* scratch = nullptr;   // device address of this device's `scratch`
  float* rope = nullptr;     // device address of this device's `rope_static`
};
constexpr int kMaxDevices = 64;
std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];
float g_rope_host[kRopeTableFloats];   // staging of the one-time table upload (no heap allocation)

// Set-up of the current device, once: the arrays' device addresses, and the RoPE table uploaded into
// rope_static (a synchronous host-to-device copy; no allocation).
hipError_t device_scratch(DeviceScratch** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceScratch& d = g_dev[dev];
  if (!d.ready) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    void* r = nullptr;
    e = hipGetSymbolAddress(&r, HIP_SYMBOL(rope_static));
    if (e != hipSuccess) return e;
    rope_table_host(1.0e4f, g_rope_host);
    e = hipMemcpy(r, g_rope_host, sizeof g_rope_host, hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
    d.scratch = p;
    d.rope = static_cast<float*>(r);
    d.ready = true;
  }
  *out = &d;
  return hipSuccess;
}

}  // namespace
}  // namespace moss

using namespace moss;

extern "C" int moss_attention_noalloc(void* qkv, void* out, int32_t batch, int32_t seq, int32_t heads,
                                      int32_t text_len, int32_t grid_w, int32_t rope, void* stream) {
  std::string msg;
  if (check_attention_args(qkv, out, batch, seq, heads, text_len, grid_w, rope, msg) != MOSS_OK) {
    thread_error() = "moss_attention_noalloc: " + msg;
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  DeviceScratch* d = nullptr;
  hipError_t e = device_scratch(&d);
  if (e != hipSuccess) {
    thread_error() = fmt("moss_attention_noalloc: set-up of the static scratch failed: %s", hipGetErrorString(e));
    return MOSS_ERR_DEVICE;
  }
  const size_t need = attention_split_workspace(batch, seq, heads);
  if (need > kScratchBytes) {
    thread_error() = fmt("moss_attention_noalloc: this shape's split tail needs %zu bytes of scratch, the static "
                         "scratch holds %zu (a chip with more than 256 compute units)", need, kScratchBytes);
    return MOSS_ERR_INVALID_ARGUMENT;
  }
  hipStream_t st = (hipStream_t)stream;
  const long D = (long)heads * kHeadDim;
  if (rope)
    e = launch_rope_inplace((uint16_t*)qkv, batch, seq, text_len, grid_w, heads, 3 * D, d->rope,
                            d->rope + kRopeMaxPos * (kHeadDim / 4), st);
  if (e == hipSuccess) {
    AttnArgs at;
    at.qkv = (const uint16_t*)qkv;
    at.out = (uint16_t*)out;
    at.B = batch;
    at.S = seq;
    at.H = heads;
    at.ld_qkv = 3 * D;
    at.ld_out = D;
    at.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)kHeadDim));
    e = launch_attention(at, st, d->scratch, kScratchBytes);
  }
  if (e != hipSuccess) {
    thread_error() = fmt("moss_attention_noalloc failed: %s", hipGetErrorString(e));
    return MOSS_ERR_DEVICE;
  }
  return MOSS_OK;
}
