// Paged decode attention for gfx950: the partition kernel (block-table gather, q.K^T,
// online softmax, P.V in fp32) and the cross-partition reduce kernel.
//
// Method: "PagedAttention and Virtual Memory Management", section 4 (block-wise
// decode with a running max / running sum, and the split across thread blocks whose
// partial (m, l, O) are combined by a second kernel); "PagedAttention: Treating KV
// Memory Like Virtual Memory", "How the kernel reads a block table" (one table lookup
// per block, a tile never straddles two blocks); "Why AI servers waste memory, and
// how paging fixes it", "Reading through the table" (only the first `valid` slots of
// the last block are read).
//
// Work decomposition.  One work-group of 4 waves owns (sequence b, KV head, partition
// p).  The partition's blocks are dealt to the waves round-robin.  Inside a wave a
// 16-token block of one KV head is read with dwordx4 loads: each lane holds 8
// consecutive elements of one token row, LPT = D/8 lanes cover a row and the wave
// covers TPI = 64/LPT tokens per load, so a block takes NI = 16/TPI loads of K and NI
// of V, each of them TPI whole rows.  q.k is v_dot2_f32_{f16,bf16} over the lane's 8
// elements followed by a DPP sum over the LPT lanes of the row.  Each row of lanes
// keeps its own running max / sum / accumulator over the tokens it sees (an online
// softmax per row); rows, then waves, are merged with the cross-block rule at the end.
// Every reduction order depends only on logical positions, so the result is
// deterministic and independent of where blocks sit in the pool.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "partition_common.h"

namespace pkv {
namespace {

template <class S, int D, int G, bool SPLIT>
__global__ __launch_bounds__(256) void pa_partition_valu(DecodeArgs a, int n_items, int per_item) {
    constexpr int LPT = D / 8;       // lanes per token row
    constexpr int TPI = 64 / LPT;    // token rows per wave load
    constexpr int NI = 16 / TPI;     // loads per block per tensor
    constexpr int W = kWavesPerGroup;
    struct Buf {
        uint4 k[NI];
        uint4 v[NI];
    };

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int r = lane / LPT;        // token row inside a load
    const int c = lane % LPT;        // 8-element chunk of the row

    const int group_id = xcd_chunked(blockIdx.x, gridDim.x, a.xcd_chunk);
    const int item = SPLIT ? group_id : group_id * W + wave;
    if (!SPLIT && item >= n_items) return;
    const Item it = decode_item(a, item, SPLIT ? 1 : per_item);
    if (it.L == 0) {
        store_empty<S, D>(a, it, G, SPLIT ? threadIdx.x : lane, SPLIT ? blockDim.x : 64);
        return;
    }
    if (it.p >= it.nparts) return;
    const int h0 = it.kvh * G;
    const size_t out_row0 = (static_cast<size_t>(it.b) * a.num_q_heads + h0) * D;

    BlockWalk walk;
    walk.init(a, it, SPLIT ? wave : 0, SPLIT ? W : 1, lane);

    uint4 qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qv[g] = *reinterpret_cast<const uint4*>(a.q + out_row0 + static_cast<size_t>(g) * D + c * 8);

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
    }

    const int row_bytes = a.row_bytes;
    const int off0 = (it.kvh * D + 8 * c) * 2 + r * row_bytes;   // + i * TPI * row_bytes

    auto load = [&](__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, Buf& buf) {
#pragma unroll
        for (int i = 0; i < NI; ++i) buf.k[i] = load16(rk, off0 + i * TPI * row_bytes);
#pragma unroll
        for (int i = 0; i < NI; ++i) buf.v[i] = load16(rv, off0 + i * TPI * row_bytes);
    };

    // merge the TPI rows of the wave (lanes with equal c) in place
    auto merge_rows = [&]() {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float M = m[g];
#pragma unroll
            for (int off = LPT; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
            const float f = (M == -INFINITY) ? 0.f : fast_exp2(m[g] - M);
            float lt = l[g] * f;
#pragma unroll
            for (int off = LPT; off < 64; off <<= 1) lt += __shfl_xor(lt, off);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float t = acc[g][e] * f;
#pragma unroll
                for (int off = LPT; off < 64; off <<= 1) t += __shfl_xor(t, off);
                acc[g][e] = t;
            }
            m[g] = M;
            l[g] = lt;
        }
    };

    // (!SPLIT) result of partition p from this wave's state, then a fresh state.  After
    // the row merge, lanes of row 0 hold elements [8c, 8c + 8) of every head; they go
    // through this wave's LDS staging area so that every lane writes whole lines.
    extern __shared__ float smem[];
    float* stage = smem + wave * G * (D + 4);     // [G][D], then (m, l) per head, 16-B aligned
    // per_item >= the partition count: this wave walks whole sequences and writes their
    // final output once, with no partial results
    const bool whole = !SPLIT && per_item >= a.num_parts;
    auto flush = [&](int p) {
        merge_rows();
        if (r == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                *reinterpret_cast<float4*>(stage + g * D + 8 * c) =
                    make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
                *reinterpret_cast<float4*>(stage + g * D + 8 * c + 4) =
                    make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
            }
            if (c == 0)
#pragma unroll
                for (int g = 0; g < G; ++g)
                    *reinterpret_cast<float2*>(stage + G * D + 2 * g) = make_float2(m[g], l[g]);
        }
        // the LDS operations of one wave complete in order: the reads below see the writes
        store_partition<S, D>(a, it, G, p, stage, stage + G * D, lane, whole);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m[g] = -INFINITY;
            l[g] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
        }
    };

    auto process = [&](int k, int valid, const Buf& buf) {
        // scores of this row's NI tokens for the G heads (base-2 units)
        float s[NI][G];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float t = S::dot2(qv[g].x, buf.k[i].x, 0.f);
                t = S::dot2(qv[g].y, buf.k[i].y, t);
                t = S::dot2(qv[g].z, buf.k[i].z, t);
                t = S::dot2(qv[g].w, buf.k[i].w, t);
                s[i][g] = group_sum<LPT>(t);
            }
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool tok_ok = (i * TPI + r) < valid;
#pragma unroll
            for (int g = 0; g < G; ++g) s[i][g] = tok_ok ? s[i][g] * a.scale_log2 : -INFINITY;
        }
        float pw[NI][G];
        float alpha[G];
        bool rescale = false;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float mb = s[0][g];
#pragma unroll
            for (int i = 1; i < NI; ++i) mb = fmaxf(mb, s[i][g]);
            const float mn = fmaxf(m[g], mb);
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            alpha[g] = fast_exp2(m[g] - mu);
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                pw[i][g] = fast_exp2(s[i][g] - mu);
                sum += pw[i][g];
            }
            l[g] = l[g] * alpha[g] + sum;
            m[g] = mn;
            rescale |= alpha[g] != 1.f;
        }
        if (__any(rescale)) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] *= alpha[g];
        }
        // P.V: rows past the valid tokens were loaded as zeros and have p = 0
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t w4[4] = {buf.v[i].x, buf.v[i].y, buf.v[i].z, buf.v[i].w};
            float vf[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                vf[2 * e] = S::lo(w4[e]);
                vf[2 * e + 1] = S::hi(w4[e]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[g][e] = fmaf(pw[i][g], vf[e], acc[g][e]);
        }
        if constexpr (!SPLIT) {     // last block of a partition (or of the sequence): emit it
            const int j = walk.jb + k;
            if (whole ? k + 1 == walk.nk : ((j + 1) % a.part_blocks == 0 || k + 1 == walk.nk))
                flush(j / a.part_blocks);
        }
    };

    walk_blocks<Buf>(a, it, walk, row_bytes, load, process);

    if constexpr (SPLIT) {
        merge_rows();
        float* sm_ml = smem;                 // [W][G][2]
        float* sm_acc = smem + W * G * 2;    // [W][G][D]
        if (r == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) sm_acc[(wave * G + g) * D + c * 8 + e] = acc[g][e];
            if (c == 0)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    sm_ml[(wave * G + g) * 2 + 0] = m[g];
                    sm_ml[(wave * G + g) * 2 + 1] = l[g];
                }
        }
        __syncthreads();
        merge_waves_and_store<S, D>(a, it, G, sm_ml, sm_acc);
    }
}

// One wave per (sequence, query head): combine the sequence's partitions,
// O = sum_k w_k acc_k / sum_k w_k l_k with w_k = 2^(m_k - max m).  Lane k holds the
// (m, l) of partition k (64 per pass); the accumulator rows are then streamed with the
// weights broadcast from those lanes, eight independent loads in flight at a time.
// The summation order is fixed (ascending k per dimension), so the result is
// deterministic.
template <class S, int D>
__global__ __launch_bounds__(256) void pa_reduce(DecodeArgs a) {
    constexpr int PER = D / 64;    // dimensions per lane
    const int lane = threadIdx.x & 63;
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= a.batch * a.num_q_heads) return;
    const int b = pair / a.num_q_heads;
    const int h = pair % a.num_q_heads;
    const int L = clamped_length(a, b);
    const int ntiles = (L + a.tile_tokens - 1) / a.tile_tokens;
    const int nparts = (ntiles + a.part_blocks - 1) / a.part_blocks;
    if (nparts <= 1) return;

    // partition k of head h = kvh*G + g is row part_row(b, kvh, k) + g: rows G apart
    const int G = a.num_q_heads / a.num_kv_heads;
    const size_t row0 = part_row(a, b, h / G, 0, G) + h % G;
    const float2* ml = reinterpret_cast<const float2*>(a.ws_ml) + row0;
    const float* acc = a.ws_acc + row0 * D + PER * lane;

    float M = -INFINITY;
    for (int k = lane; k < nparts; k += 64) M = fmaxf(M, ml[static_cast<size_t>(k) * G].x);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));

    float A[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) A[e] = 0.f;
    float lsum = 0.f;
    for (int k0 = 0; k0 < nparts; k0 += 64) {
        float w = 0.f;
        if (k0 + lane < nparts) {
            const float2 v = ml[static_cast<size_t>(k0 + lane) * G];
            w = (M == -INFINITY) ? 0.f : fast_exp2(v.x - M);
            lsum += w * v.y;
        }
        const int cnt = min(64, nparts - k0);
        const int wbits = __builtin_bit_cast(int, w);
        int i = 0;
        for (; i + 8 <= cnt; i += 8) {      // eight independent loads, then the FMAs in order
            float x[8][PER];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float* src = acc + static_cast<size_t>(k0 + i + u) * G * D;
#pragma unroll
                for (int e = 0; e < PER; ++e) x[u][e] = src[e];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, i + u));
#pragma unroll
                for (int e = 0; e < PER; ++e) A[e] = fmaf(wi, x[u][e], A[e]);
            }
        }
        for (; i < cnt; ++i) {
            const float wi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(wbits, i));
            const float* src = acc + static_cast<size_t>(k0 + i) * G * D;
#pragma unroll
            for (int e = 0; e < PER; ++e) A[e] = fmaf(wi, src[e], A[e]);
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lsum += __shfl_xor(lsum, off);
    uint16_t* o = a.out + (static_cast<size_t>(b) * a.num_q_heads + h) * D + PER * lane;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = S::narrow(lsum > 0.f ? A[e] / lsum : 0.f);
}

// The cascade reduce, one wave per (sequence, query head): the partial results of the
// batch's shared prefix (pre_parts of them, rows pair * pre_parts + s: 16-bit integers
// q with acc = q * scale, and (m, l, scale, 0)), then those of the sequence's suffix
// partitions (fp32, rows G apart as in pa_reduce; as many as its length gives, possibly
// none).  All are combined with the cross-block rule: O = sum_k w_k acc_k / sum_k w_k l_k,
// w_k = 2^(m_k - max m), an entry that saw no key (m = -inf) weighing 0.  The wave's four
// 16-lane groups take entries 4j + group (D / 16 elements per lane), up to eight entries'
// loads in flight per lane, and the groups' sums are added at the end in a fixed order:
// the result does not depend on timing.
template <class S, int D>
__global__ __launch_bounds__(256) void pa_cascade_reduce(DecodeArgs a, const int16_t* pre_acc,
                                                         const float* pre_ml, int pre_parts) {
    constexpr int PER = D / 16;    // elements per lane
    constexpr int U = 8;           // entries per lane and round
    using Raw = typename std::conditional<PER == 8, uint4, uint2>::type;   // PER int16
    const int lane = threadIdx.x & 63;
    const int grp = lane >> 4;
    const int l16 = lane & 15;
    const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= a.batch * a.num_q_heads) return;
    const int b = pair / a.num_q_heads;
    const int h = pair % a.num_q_heads;
    const int L = clamped_length(a, b);
    const int ntiles = (L + a.tile_tokens - 1) / a.tile_tokens;
    const int nsuf = (ntiles + a.part_blocks - 1) / a.part_blocks;

    const int G = a.num_q_heads / a.num_kv_heads;
    const size_t srow0 = part_row(a, b, h / G, 0, G) + h % G;
    const size_t prow0 = static_cast<size_t>(pair) * pre_parts;
    const float4* pml = reinterpret_cast<const float4*>(pre_ml) + prow0;
    const float2* sml = reinterpret_cast<const float2*>(a.ws_ml) + srow0;

    float M = -INFINITY;
    for (int k = lane; k < pre_parts; k += 64) M = fmaxf(M, pml[k].x);
    for (int k = lane; k < nsuf; k += 64) M = fmaxf(M, sml[static_cast<size_t>(k) * G].x);
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) M = fmaxf(M, __shfl_xor(M, off));
    auto weight = [&](float m) { return (M == -INFINITY || m == -INFINITY) ? 0.f : fast_exp2(m - M); };

    float A[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) A[e] = 0.f;
    float lsum = 0.f;
    // the prefix's entries
    for (int k0 = grp; k0 < pre_parts; k0 += 4 * U) {
        float4 v[U];
        Raw x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + 4 * u;
            v[u] = make_float4(-INFINITY, 0.f, 0.f, 0.f);
            x[u] = Raw{};
            if (k < pre_parts) {
                v[u] = pml[k];
                x[u] = *reinterpret_cast<const Raw*>(pre_acc + (prow0 + k) * D + PER * l16);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = weight(v[u].x);
            lsum += w * v[u].y;
            const float ws = w * v[u].z;
            const uint32_t* q = reinterpret_cast<const uint32_t*>(&x[u]);
#pragma unroll
            for (int e = 0; e < PER; e += 2) {
                const int32_t lo = static_cast<int32_t>(q[e / 2] << 16) >> 16;
                const int32_t hi = static_cast<int32_t>(q[e / 2]) >> 16;
                A[e] = fmaf(ws, static_cast<float>(lo), A[e]);
                A[e + 1] = fmaf(ws, static_cast<float>(hi), A[e + 1]);
            }
        }
    }
    // the suffix's partitions
    for (int k0 = grp; k0 < nsuf; k0 += 4 * U) {
        float2 v[U];
        float4 x[U][PER / 4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + 4 * u;
            v[u] = make_float2(-INFINITY, 0.f);
#pragma unroll
            for (int q = 0; q < PER / 4; ++q) x[u][q] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (k < nsuf) {
                v[u] = sml[static_cast<size_t>(k) * G];
                const float4* src = reinterpret_cast<const float4*>(
                    a.ws_acc + (srow0 + static_cast<size_t>(k) * G) * D + PER * l16);
#pragma unroll
                for (int q = 0; q < PER / 4; ++q) x[u][q] = src[q];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = weight(v[u].x);
            lsum += w * v[u].y;
#pragma unroll
            for (int q = 0; q < PER / 4; ++q) {
                A[4 * q] = fmaf(w, x[u][q].x, A[4 * q]);
                A[4 * q + 1] = fmaf(w, x[u][q].y, A[4 * q + 1]);
                A[4 * q + 2] = fmaf(w, x[u][q].z, A[4 * q + 2]);
                A[4 * q + 3] = fmaf(w, x[u][q].w, A[4 * q + 3]);
            }
        }
    }
    // groups (0 + 1) + (2 + 3), the same in every lane of a column
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        A[e] += __shfl_xor(A[e], 16);
        A[e] += __shfl_xor(A[e], 32);
    }
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (grp != 0) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint32_t packed[PER / 2];
#pragma unroll
    for (int e = 0; e < PER; e += 2) packed[e / 2] = S::pack2(A[e] * inv, A[e + 1] * inv);
    uint16_t* o = a.out + (static_cast<size_t>(b) * a.num_q_heads + h) * D + PER * l16;
    if constexpr (PER == 8) {
        *reinterpret_cast<uint4*>(o) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    } else {
        *reinterpret_cast<uint2*>(o) = make_uint2(packed[0], packed[1]);
    }
}

// Partitions per wave of the VALU kernel's item plan (0: the split plan is used).
template <class S, int D, int G>
int valu_parts_per_wave(const DecodeArgs& a) {
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads * a.num_parts;
    if (split_items(items)) return 0;
    static const int64_t slots = resident_waves(reinterpret_cast<const void*>(&pa_partition_valu<S, D, G, false>));
    return partitions_per_wave(items, slots, a.num_parts, a.part_blocks);
}

template <class S, int D, int G>
hipError_t launch_part_t(const DecodeArgs& a, hipStream_t stream) {
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads * a.num_parts;
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidValue;
    const size_t lds = static_cast<size_t>(kWavesPerGroup) * G * (D + 4) * sizeof(float);
    const int per = valu_parts_per_wave<S, D, G>(a);
    if (per == 0) {
        hipLaunchKernelGGL((pa_partition_valu<S, D, G, true>), dim3(static_cast<unsigned>(items)),
                           dim3(64 * kWavesPerGroup), lds, stream, a, static_cast<int>(items), 1);
    } else {
        const int64_t waves = static_cast<int64_t>(a.batch) * a.num_kv_heads * ceil_div(a.num_parts, per);
        const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
        hipLaunchKernelGGL((pa_partition_valu<S, D, G, false>), dim3(static_cast<unsigned>(groups)),
                           dim3(64 * kWavesPerGroup), lds, stream, a, static_cast<int>(waves), per);
    }
    return hipGetLastError();
}

// Partitions the VALU kernel combines by itself: all of them when each wave walks whole
// sequences, else none (1).
template <class S, int D>
int valu_chunk(int group, const DecodeArgs& a) {
    int per = 0;
    switch (group) {
        case 1: per = valu_parts_per_wave<S, D, 1>(a); break;
        case 2: per = valu_parts_per_wave<S, D, 2>(a); break;
        case 3: per = valu_parts_per_wave<S, D, 3>(a); break;
        case 4: per = valu_parts_per_wave<S, D, 4>(a); break;
        case 5: per = valu_parts_per_wave<S, D, 5>(a); break;
        case 6: per = valu_parts_per_wave<S, D, 6>(a); break;
        case 7: per = valu_parts_per_wave<S, D, 7>(a); break;
        case 8: per = valu_parts_per_wave<S, D, 8>(a); break;
        default: break;
    }
    return per >= a.num_parts ? a.num_parts : 1;
}

template <class S, int D>
hipError_t launch_part_g(int group, const DecodeArgs& a, hipStream_t stream) {
    switch (group) {
        case 1: return launch_part_t<S, D, 1>(a, stream);
        case 2: return launch_part_t<S, D, 2>(a, stream);
        case 3: return launch_part_t<S, D, 3>(a, stream);
        case 4: return launch_part_t<S, D, 4>(a, stream);
        case 5: return launch_part_t<S, D, 5>(a, stream);
        case 6: return launch_part_t<S, D, 6>(a, stream);
        case 7: return launch_part_t<S, D, 7>(a, stream);
        case 8: return launch_part_t<S, D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class S, int D>
hipError_t launch_cascade_t(const DecodeArgs& a, const int16_t* pre_acc, const float* pre_ml,
                            int pre_parts, hipStream_t stream) {
    const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;
    if (pairs <= 0) return hipSuccess;
    const int64_t groups = (pairs + 3) / 4;
    if (groups > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((pa_cascade_reduce<S, D>), dim3(static_cast<unsigned>(groups)), dim3(256), 0,
                       stream, a, pre_acc, pre_ml, pre_parts);
    return hipGetLastError();
}

template <class S, int D>
hipError_t launch_reduce_t(const DecodeArgs& a, hipStream_t stream) {
    const int64_t pairs = static_cast<int64_t>(a.batch) * a.num_q_heads;
    if (pairs <= 0 || a.num_parts <= 1) return hipSuccess;
    const int64_t groups = (pairs + 3) / 4;
    if (groups > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((pa_reduce<S, D>), dim3(static_cast<unsigned>(groups)), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

// Kernel choice: the matrix-core kernel for GQA groups of 2..16 (a real dense tile per
// block).  Single-head groups (MHA) go to it too when its group plan applies: whole
// sequences per wave and no partial results beat the VALU kernel's one wave per
// partition by several percent, and the unused matrix-core columns cost nothing in a
// kernel bound by HBM.  Otherwise (small batches) they take the VALU kernel.
// PAGEDKV_KERNEL=valu forces the VALU kernel for groups up to 8 (for comparisons);
// =mfma forces the matrix cores.
static int kernel_choice(int kv_dtype, int io_dtype, int head_dim, int group, const DecodeArgs& a) {
    if (kv_dtype == KV_DTYPE_FP8_E4M3) return 1;          // FP8 keys: matrix cores only
    const char* env = getenv("PAGEDKV_KERNEL");
    if (env && strcmp(env, "valu") == 0 && group <= kMaxGroupValu) return 0;
    if (env && strcmp(env, "mfma") == 0) return 1;
    if (group >= 2) return 1;
    return group_waves_mfma(kv_dtype, io_dtype, group, head_dim, a) > 0 ? 1 : 0;
}

int partition_chunk(int kv_dtype, int io_dtype, int head_dim, int group, const DecodeArgs& a) {
    if (kernel_choice(kv_dtype, io_dtype, head_dim, group, a) == 1)
        return partition_chunk_mfma(kv_dtype, io_dtype, group, head_dim, a);
    if (kv_dtype == KV_DTYPE_F16)
        return head_dim == 64 ? valu_chunk<F16, 64>(group, a) : valu_chunk<F16, 128>(group, a);
    return head_dim == 64 ? valu_chunk<BF16, 64>(group, a) : valu_chunk<BF16, 128>(group, a);
}

hipError_t launch_partitions(int kv_dtype, int io_dtype, int head_dim, int group,
                             const DecodeArgs& a, hipStream_t stream) {
    if (kernel_choice(kv_dtype, io_dtype, head_dim, group, a) == 1)
        return launch_partitions_mfma(kv_dtype, io_dtype, head_dim, group, a, stream);
    // the VALU kernel does not write new tokens itself: a small launch does it first
    if (a.new_k && launch_append_kv(kv_dtype, io_dtype, a, stream) != hipSuccess) return hipGetLastError();
    DecodeArgs v = a;
    v.new_k = v.new_v = nullptr;
    if (kv_dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return launch_part_g<F16, 64>(group, v, stream);
        if (head_dim == 128) return launch_part_g<F16, 128>(group, v, stream);
    } else if (kv_dtype == KV_DTYPE_BF16) {
        if (head_dim == 64) return launch_part_g<BF16, 64>(group, v, stream);
        if (head_dim == 128) return launch_part_g<BF16, 128>(group, v, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce(int io_dtype, int head_dim, const DecodeArgs& a, hipStream_t stream) {
    if (io_dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return launch_reduce_t<F16, 64>(a, stream);
        if (head_dim == 128) return launch_reduce_t<F16, 128>(a, stream);
    } else if (io_dtype == KV_DTYPE_BF16) {
        if (head_dim == 64) return launch_reduce_t<BF16, 64>(a, stream);
        if (head_dim == 128) return launch_reduce_t<BF16, 128>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_cascade_reduce(int io_dtype, int head_dim, const DecodeArgs& a,
                                 const int16_t* pre_acc, const float* pre_ml, int pre_parts,
                                 hipStream_t stream) {
    if (io_dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return launch_cascade_t<F16, 64>(a, pre_acc, pre_ml, pre_parts, stream);
        if (head_dim == 128) return launch_cascade_t<F16, 128>(a, pre_acc, pre_ml, pre_parts, stream);
    } else if (io_dtype == KV_DTYPE_BF16) {
        if (head_dim == 64) return launch_cascade_t<BF16, 64>(a, pre_acc, pre_ml, pre_parts, stream);
        if (head_dim == 128) return launch_cascade_t<BF16, 128>(a, pre_acc, pre_ml, pre_parts, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
