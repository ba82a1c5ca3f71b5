// Partition kernel on the matrix cores, for GQA groups of 2..16 query heads per KV head.
//
// Same method and work decomposition as the VALU kernel (one work-group of 4 waves per
// (sequence, KV head, 512-token partition); blocks dealt to waves round-robin; per-wave
// online softmax merged by the cross-block rule: "PagedAttention and Virtual Memory
// Management", section 4).  What changes is where the multiply-adds run.  With G query
// heads sharing a KV head, one 16-token block gives a real (16 x D) x (D x G) product
// for the scores and a (G x 16) x (16 x D) product for the values, so both go to MFMA:
//
//   scores  S^T[16 tok][16 heads] = K[16 tok][D] . Q^T[D][16 heads]   (16x16x32, D/32 ops)
//   values  O^T[D][16 heads]     += V^T[D][16 tok] . P^T[16 tok][16 heads] (16x16x16, D/16 ops)
//
// Columns >= G of Q^T are zero, so those columns are never used.  Lane l = 16c + n:
//  * K operand: token n of the block, 8 elements per MFMA (64 contiguous bytes of the
//    row per MFMA over the 4 lanes of that token).
//  * the score result puts tokens 4c..4c+3 of head n in lane (c, n) -- exactly the
//    layout of the P^T operand of the value product, so softmax needs no data movement
//    except a max across the four c-lanes of a head.
//  * V operand: lane (c, n) loads tokens 4c..4c+3 at elements [EPL*n, EPL*n + EPL)
//    (EPL = D/16), i.e. one load per token of four whole rows per wave instruction,
//    and re-packs them with v_perm into four-token columns, one per MFMA.
// Each lane keeps a partial running sum over its 4 tokens; the running max is shared
// by the head's lanes, so the accumulator rescale is uniform per head.

#include <hip/hip_runtime.h>
#include <math.h>

#include <stdlib.h>

#include <type_traits>

#include "device_common.h"

namespace pkv {
namespace {

// SPLIT = true : the 4 waves of a work-group share one (sequence, KV head, partition)
//                item, taking its blocks round-robin, and are merged through LDS.
// SPLIT = false: each wave owns a whole item (the 4 waves of a work-group take 4
//                consecutive items, i.e. 4 KV heads of the same blocks) and writes its
//                result straight from registers.  Preferred when there are enough items
//                to fill the GPU: no LDS, no barrier, and the start-up cost of a wave
//                (table fetch, first loads) is spread over the whole partition.
template <class S, int D, bool SPLIT>
__global__ __launch_bounds__(256) void pa_partition_mfma(DecodeArgs a, int G, int n_items) {
    constexpr int W = kWavesPerGroup;
    constexpr int NQK = D / 32;    // score MFMAs per block
    constexpr int EPL = D / 16;    // value MFMAs per block = V elements per lane per token
    using VRow = typename std::conditional<EPL == 8, uint4, uint2>::type;

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;

    const int group_id = xcd_order(blockIdx.x, gridDim.x);
    const int item = SPLIT ? group_id : group_id * W + wave;
    if (!SPLIT && item >= n_items) return;
    const int kvh = item % a.num_kv_heads;
    const int rest = item / a.num_kv_heads;
    const int b = rest % a.batch;
    const int p = rest / a.batch;

    int L = a.lens[b];
    L = L < 0 ? 0 : (L > a.max_blocks * kBlockSize ? a.max_blocks * kBlockSize : L);
    const int nblk = (L + kBlockSize - 1) / kBlockSize;
    const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
    const int h0 = kvh * G;
    const size_t out_row0 = (static_cast<size_t>(b) * a.num_q_heads + h0) * D;

    if (L == 0) {
        if (p == 0) {
            const int t0 = SPLIT ? threadIdx.x : lane;
            const int nt = SPLIT ? blockDim.x : 64;
            for (int i = t0; i < G * D; i += nt) a.out[out_row0 + i] = 0;
        }
        return;
    }
    if (p >= nparts) return;
    const int j0 = p * a.part_blocks;
    const int j1 = min(nblk, j0 + a.part_blocks);
    // blocks of this wave: jb + js*k for k < nk  (nk <= 256: partitions <= 4096 tokens)
    const int jb = SPLIT ? j0 + wave : j0;
    const int js = SPLIT ? W : 1;
    const int nk = j1 > jb ? (j1 - jb + js - 1) / js : 0;

    // this wave's table entries, 64 per VGPR
    const int32_t* trow = a.tables + static_cast<size_t>(b) * a.max_blocks;
    int tab[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int k = 64 * t + lane;
        tab[t] = (64 * t < nk && k < nk) ? trow[jb + js * k] : -1;
    }

    // Q^T operand: head n (zero beyond the group), 8 elements per MFMA
    uint4 qv[NQK];
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
        qv[i] = make_uint4(0, 0, 0, 0);
        if (n < G)
            qv[i] = *reinterpret_cast<const uint4*>(a.q + out_row0 + static_cast<size_t>(n) * D +
                                                    8 * (4 * i + c));
    }

    f32x4_t acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float l = 0.f;

    const int row_bytes = a.num_kv_heads * D * 2;
    const size_t blk_elems = static_cast<size_t>(a.num_kv_heads) * D * kBlockSize;
    const int koff = (kvh * D + 8 * c) * 2 + n * row_bytes;           // + 64 i
    const int voff = (kvh * D + EPL * n) * 2 + 4 * c * row_bytes;     // + r * row_bytes
    const int addr_x32 = (lane ^ 32) * 4;

    // k-th block of the wave -> (valid tokens, K and V resources covering just them)
    auto block_at = [&](int k, __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv) -> int {
        int valid = 0;
        size_t off = 0;
        if (k < nk) {
            const int kk = k & 63;
            const int t = k < 64 ? __builtin_amdgcn_readlane(tab[0], kk)
                        : k < 128 ? __builtin_amdgcn_readlane(tab[1], kk)
                        : k < 192 ? __builtin_amdgcn_readlane(tab[2], kk)
                                  : __builtin_amdgcn_readlane(tab[3], kk);
            const int j = jb + js * k;
            if (static_cast<unsigned>(t) < static_cast<unsigned>(a.num_blocks)) {
                valid = min(kBlockSize, L - j * kBlockSize);
                off = static_cast<size_t>(t) * blk_elems;
            }
        }
        rk = make_rsrc(a.k + off, valid * row_bytes);
        rv = make_rsrc(a.v + off, valid * row_bytes);
        return valid;
    };
    auto load_block = [&](__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint4 (&kk)[NQK],
                          VRow (&vv)[4]) {
#pragma unroll
        for (int i = 0; i < NQK; ++i) kk[i] = load16(rk, koff + 64 * i);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if constexpr (EPL == 8) vv[r] = load16(rv, voff + r * row_bytes);
            else vv[r] = load8(rv, voff + r * row_bytes);
        }
    };

    auto process = [&](int valid, const uint4 (&kk)[NQK], const VRow (&vv)[4]) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NQK; ++i) s = S::mfma_k32(kk[i], qv[i], s);
        float sr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sr[r] = (4 * c + r < valid) ? s[r] * a.scale_log2 : -INFINITY;
        float mb = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
        mb = fmaxf(mb, xor16(mb));
        mb = fmaxf(mb, xor32(mb, addr_x32));
        const float mn = fmaxf(m, mb);
        const float mu = (mn == -INFINITY) ? 0.f : mn;
        const float alpha = fast_exp2(m - mu);
        float pr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sr[r] - mu);
        l = l * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
        m = mn;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
        }
        const uint2 pt = make_uint2(S::pack2(pr[0], pr[1]), S::pack2(pr[2], pr[3]));
        // V^T operand of element e: (tok 4c, 4c+1 | 4c+2, 4c+3) at element EPL*n + e;
        // rows past the valid tokens were loaded as zeros
        uint32_t w0[EPL / 2], w1[EPL / 2], w2[EPL / 2], w3[EPL / 2];
        if constexpr (EPL == 8) {
            w0[0] = vv[0].x; w0[1] = vv[0].y; w0[2] = vv[0].z; w0[3] = vv[0].w;
            w1[0] = vv[1].x; w1[1] = vv[1].y; w1[2] = vv[1].z; w1[3] = vv[1].w;
            w2[0] = vv[2].x; w2[1] = vv[2].y; w2[2] = vv[2].z; w2[3] = vv[2].w;
            w3[0] = vv[3].x; w3[1] = vv[3].y; w3[2] = vv[3].z; w3[3] = vv[3].w;
        } else {
            w0[0] = vv[0].x; w0[1] = vv[0].y;
            w1[0] = vv[1].x; w1[1] = vv[1].y;
            w2[0] = vv[2].x; w2[1] = vv[2].y;
            w3[0] = vv[3].x; w3[1] = vv[3].y;
        }
#pragma unroll
        for (int k = 0; k < EPL / 2; ++k) {
            const uint2 even = make_uint2(lo_halves(w0[k], w1[k]), lo_halves(w2[k], w3[k]));
            const uint2 odd = make_uint2(hi_halves(w0[k], w1[k]), hi_halves(w2[k], w3[k]));
            acc[2 * k] = S::mfma_k16(even, pt, acc[2 * k]);
            acc[2 * k + 1] = S::mfma_k16(odd, pt, acc[2 * k + 1]);
        }
    };

    // Two register sets, alternating.  Every iteration issues exactly one block's loads
    // (an empty resource past the wave's last block), so the wait before computing a
    // block always leaves the following block's loads in flight.
    uint4 ka[NQK], kb[NQK];
    VRow va[4], vb[4];
    __amdgpu_buffer_rsrc_t rk, rv;
    int valid_a = block_at(0, rk, rv);
    load_block(rk, rv, ka, va);
    for (int k = 0; k < nk; k += 2) {
        const int valid_b = block_at(k + 1, rk, rv);
        load_block(rk, rv, kb, vb);
        process(valid_a, ka, va);
        if (k + 1 >= nk) break;
        valid_a = block_at(k + 2, rk, rv);
        load_block(rk, rv, ka, va);
        process(valid_b, kb, vb);
    }

    // per-head totals: the four c-lanes of head n hold partial sums of l
    l += xor16(l);
    l += xor32(l, addr_x32);

    if constexpr (!SPLIT) {
        // lane (c, n) holds dims EPL*(4c + r) + e of head n: EPL contiguous values per r
        if (n < G) {
            const size_t h = static_cast<size_t>(h0 + n);
            if (nparts == 1) {
                uint16_t* o = a.out + (static_cast<size_t>(b) * a.num_q_heads + h) * D;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint32_t wv[EPL / 2];
#pragma unroll
                    for (int e = 0; e < EPL / 2; ++e)
                        wv[e] = static_cast<uint32_t>(S::narrow(l > 0.f ? acc[2 * e][r] / l : 0.f)) |
                                (static_cast<uint32_t>(S::narrow(l > 0.f ? acc[2 * e + 1][r] / l : 0.f)) << 16);
                    uint16_t* dst = o + EPL * (4 * c + r);
                    if constexpr (EPL == 8) *reinterpret_cast<uint4*>(dst) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                    else *reinterpret_cast<uint2*>(dst) = make_uint2(wv[0], wv[1]);
                }
            } else {
                const size_t ph = (static_cast<size_t>(b) * a.num_q_heads + h) * a.num_parts + p;
                float* wa = a.ws_acc + ph * D;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float* dst = wa + EPL * (4 * c + r);
#pragma unroll
                    for (int e = 0; e < EPL; e += 4)
                        *reinterpret_cast<float4*>(dst + e) =
                            make_float4(acc[e][r], acc[e + 1][r], acc[e + 2][r], acc[e + 3][r]);
                }
                if (c == 0) *reinterpret_cast<float2*>(a.ws_ml + ph * 2) = make_float2(m, l);
            }
        }
    } else {
        extern __shared__ float smem[];
        float* sm_ml = smem;                 // [W][G][2]
        float* sm_acc = smem + W * G * 2;    // [W][G][D]
        if (n < G) {
            float* dst = sm_acc + (wave * G + n) * D;
#pragma unroll
            for (int e = 0; e < EPL; ++e)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[EPL * (4 * c + r) + e] = acc[e][r];
            if (c == 0) {
                sm_ml[(wave * G + n) * 2 + 0] = m;
                sm_ml[(wave * G + n) * 2 + 1] = l;
            }
        }
        __syncthreads();

        for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
            const int g = idx / D;
            const int dd = idx % D;
            float M = sm_ml[g * 2];
#pragma unroll
            for (int w = 1; w < W; ++w) M = fmaxf(M, sm_ml[(w * G + g) * 2]);
            float lsum = 0.f, A = 0.f;
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float mw = sm_ml[(w * G + g) * 2];
                const float f = (M == -INFINITY) ? 0.f : fast_exp2(mw - M);
                lsum += f * sm_ml[(w * G + g) * 2 + 1];
                A += f * sm_acc[(w * G + g) * D + dd];
            }
            if (nparts == 1) {
                a.out[out_row0 + idx] = S::narrow(lsum > 0.f ? A / lsum : 0.f);
            } else {
                const size_t ph = (static_cast<size_t>(b) * a.num_q_heads + h0 + g) * a.num_parts + p;
                a.ws_acc[ph * D + dd] = A;
                if (dd == 0) {
                    a.ws_ml[ph * 2 + 0] = M;
                    a.ws_ml[ph * 2 + 1] = lsum;
                }
            }
        }
    }
}

// One wave per item once there are enough items to fill the GPU several times over.
static bool use_split(int64_t items) {
    const char* env = getenv("PAGEDKV_SPLIT");
    if (env) return env[0] == '1';
    return items < 4096;
}

template <class S, int D>
hipError_t launch_t(int group, const DecodeArgs& a, hipStream_t stream) {
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads * a.num_parts;
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidValue;
    if (use_split(items)) {
        const size_t lds = static_cast<size_t>(kWavesPerGroup) * group * (D + 2) * sizeof(float);
        hipLaunchKernelGGL((pa_partition_mfma<S, D, true>), dim3(static_cast<unsigned>(items)),
                           dim3(64 * kWavesPerGroup), lds, stream, a, group, static_cast<int>(items));
    } else {
        const int64_t groups = (items + kWavesPerGroup - 1) / kWavesPerGroup;
        hipLaunchKernelGGL((pa_partition_mfma<S, D, false>), dim3(static_cast<unsigned>(groups)),
                           dim3(64 * kWavesPerGroup), 0, stream, a, group, static_cast<int>(items));
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_partitions_mfma(int dtype, int head_dim, int group, const DecodeArgs& a,
                                  hipStream_t stream) {
    if (group < 1 || group > 16) return hipErrorInvalidValue;
    if (dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return launch_t<F16, 64>(group, a, stream);
        if (head_dim == 128) return launch_t<F16, 128>(group, a, stream);
    } else if (dtype == KV_DTYPE_BF16) {
        if (head_dim == 64) return launch_t<BF16, 64>(group, a, stream);
        if (head_dim == 128) return launch_t<BF16, 128>(group, a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
