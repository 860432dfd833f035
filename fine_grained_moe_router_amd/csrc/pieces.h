// pieces.h -- register-held row pieces of FP8 GEMVs at batch 1..8 (gfx950): a workgroup's
// rows read in 16-byte pieces by 16, 32 or 64 lanes per row, every piece requested before
// the vector-dependent work, dotted against bf16 or fp32 vectors staged in LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "handoff.h"

namespace moe {
namespace dev {

// A workgroup's rows of an FP8 matrix [N][K] (K a multiple of 16 LPR): LPR lanes per row,
// 256 / LPR rows per workgroup; lane li of a row's group holds the row's 16-byte pieces
// li, li + LPR, ... (ch = K / (16 LPR) <= MAXCH of them). load() issues every piece at
// once, ahead of the vector-dependent work, so the weight stream overlaps it.
template <int LPR, int MAXCH>
struct Pieces {
    uint4 q[MAXCH];
    __device__ __forceinline__ void load(const uint8_t *row, int li, int ch) {
#pragma unroll
        for (int k = 0; k < MAXCH; ++k)
            if (k < ch) q[k] = ld16nt(row + (size_t)(k * LPR + li) * 16);
    }
    // sum_c dec(Q[c]) x[c] over this lane's pieces, x bf16 in LDS (two uint4 per piece)
    __device__ __forceinline__ float dot_bf16(const uint4 *xs, int li, int ch) const {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < MAXCH; ++k)
            if (k < ch) {
                bf16x2 w[8];
                decode16_bf16(q[k], w);
                const int p = (k * LPR + li) * 2;
                acc = dot16(w, xs[p], xs[p + 1], acc);
            }
        return acc;
    }
    // the same with an fp32 vector in LDS (four float4 per piece)
    __device__ __forceinline__ float dot_f32(const float4 *hs, int li, int ch) const {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < MAXCH; ++k)
            if (k < ch) {
                const uint32_t qw[4] = {q[k].x, q[k].y, q[k].z, q[k].w};
                const float4 *hp = hs + (k * LPR + li) * 4;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const f32x2 lo = fp8x2_to_f32<false>(qw[u]), hi = fp8x2_to_f32<true>(qw[u]);
                    const float4 hv = hp[u];
                    acc = fmaf(lo.x, hv.x, acc);
                    acc = fmaf(lo.y, hv.y, acc);
                    acc = fmaf(hi.x, hv.z, acc);
                    acc = fmaf(hi.y, hv.w, acc);
                }
            }
        return acc;
    }
};

// Sum over a row's LPR lanes (aligned groups of a wave); every lane of the group gets it.
template <int LPR>
__device__ __forceinline__ float group_sum(float v) {
    v = row16_sum(v);
    if (LPR >= 32) v += __shfl_xor(v, 16);
    if (LPR >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Copy n 16-byte words from global memory into LDS, four words a thread at a time: the
// four loads are issued before the first store, so they are in flight together.
__device__ __forceinline__ void stage16(uint4 *dst, const uint4 *src, int n) {
    for (int b = threadIdx.x; b < n; b += 1024) {
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = src[min(b + 256 * i, n - 1)];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (b + 256 * i < n) dst[b + 256 * i] = v[i];
    }
}

}  // namespace dev
}  // namespace moe
