// lcd_probe.hip -- a plain streaming read, for measurement only: the
// practical HBM read ceiling at a given byte count on the running GPU, against
// which the scan kernels' bandwidth is judged.  Each workgroup reads a
// contiguous share of the buffer with 16-byte loads (four in flight per lane)
// and writes one float, so its traffic is the buffer read once.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"

namespace lcd {
namespace {

constexpr int kProbeThreads = 256;

__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const float4 *__restrict__ buf, int64_t n4, int64_t per_block,
                  float *__restrict__ out) {
    const int64_t b0 = blockIdx.x * per_block;
    const int64_t b1 = b0 + per_block < n4 ? b0 + per_block : n4;
    float s = 0.0f;
    for (int64_t i = b0 + threadIdx.x; i < b1; i += 4 * kProbeThreads) {
        float4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t j = i + k * kProbeThreads;
            v[k] = j < b1 ? buf[j] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) s += v[k].x + v[k].y + v[k].z + v[k].w;
    }
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    __shared__ float w[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = w[0] + w[1] + w[2] + w[3];
}

}  // namespace
}  // namespace lcd

extern "C" int lcd_read_probe(const void *buf, int64_t bytes, int32_t blocks, float *out,
                              void *stream, void *ev_start, void *ev_stop) {
    using namespace lcd;
    if (!buf || !out || bytes < 16 || blocks < 1 || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return LCD_EINVAL;
    const int64_t n4 = bytes / 16;
    const int64_t per_block = (n4 + blocks - 1) / blocks;
    hipExtLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0u,
                          reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(ev_start),
                          reinterpret_cast<hipEvent_t>(ev_stop), 0u,
                          static_cast<const float4 *>(buf), n4, per_block, out);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}
