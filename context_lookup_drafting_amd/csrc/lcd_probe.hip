// lcd_probe.hip -- measurement kernels: a plain streaming read and an empty
// kernel, each with GPU-stamped events, giving the practical HBM read ceiling
// at a byte count and the floor of one launch on the running GPU, against
// which the scan kernels are judged.
//
// The read streams the buffer once with 16-byte loads (a wave-wide load moves
// 1 KiB, coalesced), `depth` loads in flight per lane, and either gives each
// workgroup one contiguous share of the buffer or interleaves the workgroups
// over blocks of 256 x depth granules (grid-stride), with plain or
// non-temporal loads (the scan and the sampled verification stream theirs
// non-temporal).  Every workgroup writes one word, so the traffic is the
// buffer read once.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcd.h"

namespace lcd {
namespace {

constexpr int kProbeThreads = 256;

typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int4 load_nt(const int4 *p) {
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
    return make_int4(v.x, v.y, v.z, v.w);
}

template <int kDepth, bool kInterleave, bool kNT>
__global__ void __launch_bounds__(kProbeThreads)
read_probe_kernel(const int4 *__restrict__ buf, int64_t n16, int64_t per_block,
                  int32_t *__restrict__ out) {
    int acc = 0;
    constexpr int64_t kStep = (int64_t)kProbeThreads * kDepth;     // granules per round
    int64_t b0, b1, stride;
    if (kInterleave) {
        b0 = (int64_t)blockIdx.x * kStep;
        b1 = n16;
        stride = (int64_t)gridDim.x * kStep;
    } else {
        b0 = (int64_t)blockIdx.x * per_block;
        b1 = b0 + per_block < n16 ? b0 + per_block : n16;
        stride = kStep;
    }
    for (int64_t i = b0 + threadIdx.x; i < b1; i += stride) {
        int4 v[kDepth];
#pragma unroll
        for (int k = 0; k < kDepth; ++k) {
            const int64_t j = i + (int64_t)k * kProbeThreads;
            v[k] = j < b1 ? (kNT ? load_nt(buf + j) : buf[j]) : make_int4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kDepth; ++k) acc += (v[k].x ^ v[k].y) + (v[k].z ^ v[k].w);
    }
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    __shared__ int w[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = w[0] + w[1] + w[2] + w[3];
}

__global__ void __launch_bounds__(kProbeThreads) empty_probe_kernel() {}

template <int kDepth, bool kInterleave, bool kNT>
hipError_t launch_read(const void *buf, int64_t n16, int32_t blocks, int32_t *out, hipStream_t st,
                       hipEvent_t ev0, hipEvent_t ev1) {
    const int64_t per_block = (n16 + blocks - 1) / blocks;
    hipExtLaunchKernelGGL(read_probe_kernel<kDepth, kInterleave, kNT>, dim3((unsigned)blocks),
                          dim3(kProbeThreads), 0u, st, ev0, ev1, 0u,
                          static_cast<const int4 *>(buf), n16, per_block, out);
    return hipGetLastError();
}

}  // namespace
}  // namespace lcd

extern "C" int lcd_read_probe(const void *buf, int64_t bytes, int32_t blocks, int32_t variant,
                              int32_t *out, void *stream, void *ev_start, void *ev_stop) {
    using namespace lcd;
    if (!buf || !out || bytes < 16 || blocks < 1 || blocks > (1 << 20) || (bytes & 15) != 0 ||
        (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return LCD_EINVAL;
    const int64_t n16 = bytes / 16;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const hipEvent_t e0 = reinterpret_cast<hipEvent_t>(ev_start);
    const hipEvent_t e1 = reinterpret_cast<hipEvent_t>(ev_stop);
    hipError_t err;
    const bool nt = (variant & LCD_PROBE_NT) != 0;
    switch (variant & ~LCD_PROBE_NT) {
    case LCD_PROBE_CONTIG_4:
        err = nt ? launch_read<4, false, true>(buf, n16, blocks, out, st, e0, e1)
                 : launch_read<4, false, false>(buf, n16, blocks, out, st, e0, e1);
        break;
    case LCD_PROBE_CONTIG_8:
        err = nt ? launch_read<8, false, true>(buf, n16, blocks, out, st, e0, e1)
                 : launch_read<8, false, false>(buf, n16, blocks, out, st, e0, e1);
        break;
    case LCD_PROBE_INTERLEAVE_4:
        err = nt ? launch_read<4, true, true>(buf, n16, blocks, out, st, e0, e1)
                 : launch_read<4, true, false>(buf, n16, blocks, out, st, e0, e1);
        break;
    case LCD_PROBE_INTERLEAVE_8:
        err = nt ? launch_read<8, true, true>(buf, n16, blocks, out, st, e0, e1)
                 : launch_read<8, true, false>(buf, n16, blocks, out, st, e0, e1);
        break;
    case LCD_PROBE_INTERLEAVE_16:
        err = nt ? launch_read<16, true, true>(buf, n16, blocks, out, st, e0, e1)
                 : launch_read<16, true, false>(buf, n16, blocks, out, st, e0, e1);
        break;
    default: return LCD_EINVAL;
    }
    return err == hipSuccess ? LCD_OK : LCD_EHIP;
}

extern "C" int lcd_empty_probe(int32_t blocks, void *stream, void *ev_start, void *ev_stop) {
    using namespace lcd;
    if (blocks < 1 || blocks > (1 << 20)) return LCD_EINVAL;
    hipExtLaunchKernelGGL(empty_probe_kernel, dim3((unsigned)blocks), dim3(kProbeThreads), 0u,
                          reinterpret_cast<hipStream_t>(stream), reinterpret_cast<hipEvent_t>(ev_start),
                          reinterpret_cast<hipEvent_t>(ev_stop), 0u);
    return hipGetLastError() == hipSuccess ? LCD_OK : LCD_EHIP;
}
