// Diagnostic: the HBM read rate of a plain streaming kernel on this device, the practical
// ceiling the GEMV's bandwidth is read against.  Each wavefront reads contiguous runs of
// 4 KB (four 16-byte nontemporal loads per lane, one 1 KB piece each, all in flight), runs
// strided over the grid, and folds what it reads into one word; each workgroup writes one
// word, so the writes are negligible next to the reads.  (Measured on MI355X: wave-contiguous
// runs with nontemporal loads read ~7.0 TB/s; a lane-strided grid loop ~6.2; plain loads ~6.2.)
#include "gale_internal.h"

namespace gale {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kReadRun = 4;   // 1 KB pieces per wavefront step

__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  __shared__ uint32_t s_acc[4];
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * 4;
  uint32_t acc = 0;
  // whole runs: granules [0, n_runs * 64 * kReadRun)
  for (int64_t base = wave * 64 * kReadRun; base + 64 * kReadRun <= n16; base += nw * 64 * kReadRun) {
    u32x4_t v[kReadRun];
#pragma unroll
    for (int u = 0; u < kReadRun; ++u) v[u] = __builtin_nontemporal_load(src + base + 64 * u + lane);
#pragma unroll
    for (int u = 0; u < kReadRun; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // the ragged tail, granule by granule
  for (int64_t i = (n16 / (64 * kReadRun)) * (64 * kReadRun) + wave * 64 + lane; i < n16; i += nw * 64) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
  if (lane == 0) s_acc[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s_acc[0] ^ s_acc[1] ^ s_acc[2] ^ s_acc[3];
}

}  // namespace gale

using namespace gale;

extern "C" int gale_read_stream(const void* src, size_t bytes, uint32_t* sink, int32_t sink_words,
                                hipStream_t stream) {
  if (!src || !sink) {
    set_error("gale_read_stream: src and sink must be set");
    return GALE_ERR_NULL;
  }
  if (bytes == 0 || bytes % 16 != 0 || sink_words < 1) {
    set_error("gale_read_stream: bytes=%zu must be a positive multiple of 16, sink_words=%d positive", bytes,
              (int)sink_words);
    return GALE_ERR_SHAPE;
  }
  if (((uintptr_t)src & 15) != 0 || ((uintptr_t)sink & 3) != 0) {
    set_error("gale_read_stream: src must be 16-byte aligned and sink 4-byte aligned");
    return GALE_ERR_ALIGN;
  }
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t grid = (n16 + 255) / 256;
  if (grid > sink_words) grid = sink_words;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(src), n16, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("gale_read_stream: %s", hipGetErrorString(e));
    return GALE_ERR_HIP;
  }
  return GALE_OK;
}
