// Partition kernel on the matrix cores, for GQA groups of 1..16 query heads per KV head.
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
//
// FP8 keys and values (KV8): a lane loads the E4M3 codes it needs as whole 16-byte (K)
// and 8- or 4-byte (V) pieces and widens them exactly to the query's 16-bit type in
// registers (two values per instruction), so the matrix-core products above run
// unchanged.  For the score product the lane of column group c then supplies the
// contiguous elements [c D/4, (c+1) D/4) of its token, 8 per MFMA; Q^T is loaded with
// the same assignment (the contraction does not care which lane supplies which k).

#include <hip/hip_runtime.h>
#include <math.h>

#include <stdlib.h>

#include <type_traits>

#include "partition_common.h"

namespace pkv {
namespace {

// Three ways to map (sequence, KV head, partition) items onto waves:
//  kSplit : the 4 waves of a work-group share one item, taking its blocks
//           round-robin, merged through LDS.  For small problems.
//  kItem  : each wave owns whole items (one or more consecutive partitions, walked as
//           one stream) and writes each partition's partial result to the workspace;
//           a second kernel combines the partitions.
//  kGroup : a work-group owns a chunk of `per_item` consecutive partitions of `heads`
//           consecutive KV heads of one sequence, with blockDim / 64 / heads waves
//           ("slots") per head; each wave walks `ppw` consecutive partitions of its head
//           as one stream, leaves its state in LDS, and the work-group combines the
//           slots of each head with the cross-block rule.  A sequence that fits in one
//           chunk gets its final output right away: no partial results go to HBM and no
//           second kernel runs.
enum Mode { kSplit = 0, kItem = 1, kGroup = 2 };

// kGroup: the blocks of chunk c (partitions [c * chunk, (c + 1) * chunk)) that slot
// `slot` of KV head kvh of sequence b walks: partitions [p, p_end), possibly none.
__device__ __forceinline__ Item group_item(const DecodeArgs& a, int b, int kvh, int c, int chunk,
                                           int slot, int ppw) {
    Item it;
    it.b = b;
    it.kvh = kvh;
    it.L = clamped_length(a, b);
    const int ntiles = (it.L + a.tile_tokens - 1) / a.tile_tokens;
    it.nparts = (ntiles + a.part_blocks - 1) / a.part_blocks;
    const int chunk_end = min(it.nparts, (c + 1) * chunk);
    it.p = c * chunk + slot * ppw;
    it.p_end = max(it.p, min(chunk_end, it.p + ppw));
    it.j0 = min(ntiles, it.p * a.part_blocks);
    it.j1 = min(ntiles, it.p_end * a.part_blocks);
    return it;
}

template <bool KV8, int NQK, int EPL> struct KVBuf;
template <int NQK, int EPL> struct KVBuf<false, NQK, EPL> {      // 16-bit K and V
    uint4 k[NQK];
    typename std::conditional<EPL == 8, uint4, uint2>::type v[4];
};
template <int NQK, int EPL> struct KVBuf<true, NQK, EPL> {       // E4M3 codes
    uint4 k[NQK / 2];
    typename std::conditional<EPL == 8, uint2, uint32_t>::type v[4];
};

// 8-token blocks, two per 16-row tile.  With B = 8 a tile of one block fills half of the
// matrix-core tile; pairing blocks 2k and 2k + 1 of a wave's range fills it and halves
// the walk.  Rows 0-7 of the tile come from the first block, rows 8-15 from the second,
// so each lane addresses its own block: through one buffer resource over the whole
// layer (32-bit offsets, hence layers up to 0x7FF00000 bytes), with an offset past its end for a
// row that is not there (beyond the length or an entry outside the pool), which loads
// zeros.  The tile's valid rows are still a prefix: the second block only holds tokens
// when the first is full.
struct PairLoc {
    int off0, off1;      // byte offsets of the two blocks in the layer (-1: none)
    int valid0, valid1;  // tokens in each
};

struct PairWalk {
    int jb, j_end, nk;   // first tile (even), end, number of pairs
    int tab0[4], tab1[4];

    __device__ __forceinline__ void init_range(const DecodeArgs& a, const Item& it, int j_begin,
                                               int j_stop, int lane) {
        jb = j_begin;
        j_end = j_stop;
        nk = j_stop > j_begin ? (j_stop - j_begin + 1) / 2 : 0;
        const int32_t* trow = a.tables + static_cast<size_t>(it.b) * a.table_stride;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k = 64 * t + lane;
            const int j = jb + 2 * k;
            tab0[t] = (64 * t < nk && k < nk) ? trow[j] : -1;
            tab1[t] = (64 * t < nk && k < nk && j + 1 < j_stop) ? trow[j + 1] : -1;
        }
    }

    __device__ __forceinline__ int at(const DecodeArgs& a, const Item& it, int k, PairLoc& loc) const {
        int t0 = -1, t1 = -1;
        if (k < nk) {
            const int kk = k & 63;
            t0 = k < 64 ? __builtin_amdgcn_readlane(tab0[0], kk)
               : k < 128 ? __builtin_amdgcn_readlane(tab0[1], kk)
               : k < 192 ? __builtin_amdgcn_readlane(tab0[2], kk)
                         : __builtin_amdgcn_readlane(tab0[3], kk);
            t1 = k < 64 ? __builtin_amdgcn_readlane(tab1[0], kk)
               : k < 128 ? __builtin_amdgcn_readlane(tab1[1], kk)
               : k < 192 ? __builtin_amdgcn_readlane(tab1[2], kk)
                         : __builtin_amdgcn_readlane(tab1[3], kk);
        }
        const int j = jb + 2 * k;
        const int block_bytes = 8 * a.row_bytes;
        const bool ok0 = static_cast<unsigned>(t0) < static_cast<unsigned>(a.num_blocks);
        const bool ok1 = static_cast<unsigned>(t1) < static_cast<unsigned>(a.num_blocks);
        loc.valid0 = uniform(ok0 ? max(0, min(8, it.L - 8 * j)) : 0);
        loc.valid1 = uniform(ok1 && loc.valid0 == 8 ? max(0, min(8, it.L - 8 * (j + 1))) : 0);
        loc.off0 = uniform(ok0 ? t0 * block_bytes : -1);
        loc.off1 = uniform(ok1 ? t1 * block_bytes : -1);
        return loc.valid0 + loc.valid1;
    }
};

// walk_blocks3's schedule over tile pairs
template <class Buf, class Load, class Process>
__device__ __forceinline__ void walk_pairs3(const DecodeArgs& a, const Item& it, const PairWalk& w,
                                            Load load, Process process) {
    Buf b0, b1, b2;
    PairLoc loc;
    int v0 = w.at(a, it, 0, loc);
    load(loc, b0);
    int v1 = w.at(a, it, 1, loc);
    load(loc, b1);
    for (int k = 0; k < w.nk; k += 3) {
        const int v2 = w.at(a, it, k + 2, loc);
        load(loc, b2);
        __builtin_amdgcn_sched_barrier(0);
        process(k, v0, b0);
        if (k + 1 >= w.nk) break;
        v0 = w.at(a, it, k + 3, loc);
        load(loc, b0);
        __builtin_amdgcn_sched_barrier(0);
        process(k + 1, v1, b1);
        if (k + 2 >= w.nk) break;
        v1 = w.at(a, it, k + 4, loc);
        load(loc, b1);
        __builtin_amdgcn_sched_barrier(0);
        process(k + 2, v2, b2);
    }
}

// The decode step's new token (position L - 1) of KV head kvh into the slot its table
// entry gives it: written by the wave that reads that tile, before its walk, and waited
// for, so the wave's own loads of the tile see it (no other wave reads the tile; the
// L1 of this compute unit holds no copy of it, as nothing read it in this launch).
template <class S, int D, bool KV8>
__device__ __forceinline__ void append_token(const DecodeArgs& a, int b, int kvh, int L, int lane) {
    const int last = L - 1;
    const int blk = a.tables[static_cast<size_t>(b) * a.table_stride + last / a.block_size];
    if (static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks) && lane < D / 2) {
        const size_t slot = static_cast<size_t>(blk) * a.block_size + last % a.block_size;
        const size_t src = (static_cast<size_t>(b) * a.num_kv_heads + kvh) * (D / 2) + lane;
        const uint32_t kw = reinterpret_cast<const uint32_t*>(a.new_k)[src];
        const uint32_t vw = reinterpret_cast<const uint32_t*>(a.new_v)[src];
        if constexpr (KV8) {
            const size_t dst = slot * a.row_bytes + kvh * D + 2 * lane;
            *reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a.k) + dst) =
                static_cast<uint16_t>(fp8x2_from(S::lo(kw), S::hi(kw)));
            *reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(a.v) + dst) =
                static_cast<uint16_t>(fp8x2_from(S::lo(vw), S::hi(vw)));
        } else {
            const size_t dst = slot * a.row_bytes + (kvh * D + 2 * lane) * 2;
            *reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(a.k) + dst) = kw;
            *reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(a.v) + dst) = vw;
        }
    }
    // the stores complete before any load below is issued
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The batch's sequences longest first, for the group plan's work-groups: a counting sort
// of the lengths in tiles, scaled into kOrderBuckets keys, in one work-group.  Sequences
// with equal keys land in an unspecified order among themselves; which work-group takes a
// sequence changes no result.
constexpr int kOrderThreads = 1024;
constexpr int kOrderBuckets = 2 * kOrderThreads;
__global__ __launch_bounds__(kOrderThreads) void pa_length_order(DecodeArgs a, int32_t* order) {
    __shared__ int start[kOrderBuckets];
    __shared__ int scan[kOrderThreads];
    const int tid = threadIdx.x;
    const int64_t max_tiles = static_cast<int64_t>(a.max_blocks) << a.tiles_log2;
    auto key = [&](int b) {                      // 0 for the longest
        const int64_t tiles = (clamped_length(a, b) + a.tile_tokens - 1) / a.tile_tokens;
        const int64_t k = tiles * (kOrderBuckets - 1) / (max_tiles > 0 ? max_tiles : 1);
        return kOrderBuckets - 1 - static_cast<int>(k < kOrderBuckets - 1 ? k : kOrderBuckets - 1);
    };
    for (int i = tid; i < kOrderBuckets; i += kOrderThreads) start[i] = 0;
    __syncthreads();
    for (int b = tid; b < a.batch; b += kOrderThreads) atomicAdd(&start[key(b)], 1);
    __syncthreads();
    // exclusive prefix sum over the buckets, two per thread
    const int h0 = start[2 * tid];
    const int own = h0 + start[2 * tid + 1];
    scan[tid] = own;
    __syncthreads();
    for (int off = 1; off < kOrderThreads; off <<= 1) {
        const int v = tid >= off ? scan[tid - off] : 0;
        __syncthreads();
        scan[tid] += v;
        __syncthreads();
    }
    const int before = scan[tid] - own;
    start[2 * tid] = before;
    start[2 * tid + 1] = before + h0;
    __syncthreads();
    for (int b = tid; b < a.batch; b += kOrderThreads) order[atomicAdd(&start[key(b)], 1)] = b;
}

template <class S, int D, int MODE, bool NT, bool KV8, bool PAIR = false>
__global__ __launch_bounds__(512) void pa_partition_mfma(DecodeArgs a, int G, int n_items,
                                                         int per_item, int ppw, int heads) {
    static_assert(!PAIR || MODE == kGroup, "paired 8-token blocks only in the group plan");
    constexpr bool SPLIT = MODE == kSplit;
    constexpr int W = kWavesPerGroup;
    constexpr int NQK = D / 32;    // score MFMAs per block
    constexpr int EPL = D / 16;    // value MFMAs per block = V elements per lane per token
    using Buf = KVBuf<KV8, NQK, EPL>;

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;

    const int group_id = xcd_chunked(blockIdx.x, gridDim.x, a.xcd_chunk);
    Item it;
    int chunk_id = 0;
    if constexpr (MODE == kGroup) {
        // work-group -> (KV heads [kvh0, kvh0 + heads), sequence, chunk); wave -> (head, slot)
        const int ngrp = a.num_kv_heads / heads;
        const int rest = group_id / ngrp;
        chunk_id = rest / a.batch;
        const int b = a.order ? a.order[rest % a.batch] : rest % a.batch;
        it = group_item(a, b, (group_id % ngrp) * heads + wave % heads, chunk_id, per_item,
                        wave / heads, ppw);
        // both exits below are the same for the whole work-group (same sequence, chunk)
        if (it.L == 0) {
            if (it.p == 0) store_empty<S, D>(a, it, G, lane, 64);
            return;
        }
        if (chunk_id * per_item >= it.nparts) return;
    } else {
        const int item = MODE == kItem ? group_id * W + wave : group_id;
        if (MODE == kItem && item >= n_items) return;
        it = decode_item(a, item, SPLIT ? 1 : per_item);
        if (it.L == 0) {
            store_empty<S, D>(a, it, G, SPLIT ? threadIdx.x : lane, SPLIT ? blockDim.x : 64);
            return;
        }
        if (it.p >= it.nparts) return;
    }
    const int h0 = it.kvh * G;
    const size_t out_row0 = (static_cast<size_t>(it.b) * a.num_q_heads + h0) * D;

    BlockWalk walk;
    if constexpr (MODE == kGroup) {
        walk.init_range(a, it, it.j0, it.j1, lane);
    } else {
        walk.init(a, it, SPLIT ? wave : 0, SPLIT ? W : 1, lane);
    }

    // Q^T operand: head n (zero beyond the group), 8 elements per MFMA: elements
    // 8 (4i + c) for 16-bit keys, c D/4 + 8i for FP8 keys (matching the K operand)
    uint4 qv[NQK];
#pragma unroll
    for (int i = 0; i < NQK; ++i) {
        qv[i] = make_uint4(0, 0, 0, 0);
        const int e0 = KV8 ? c * (D / 4) + 8 * i : 8 * (4 * i + c);
        if (n < G)
            qv[i] = *reinterpret_cast<const uint4*>(a.q + out_row0 + static_cast<size_t>(n) * D + e0);
    }

    // The table entries and Q must be in registers before the first block can be
    // addressed anyway; waiting for them here also tells the compiler that none of
    // the loads below have to wait for them again.
    __builtin_amdgcn_s_waitcnt(0);

    f32x4_t acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY;
    float l = 0.f;

    const int row_bytes = a.row_bytes;
    constexpr int EB = KV8 ? 1 : 2;                                       // bytes per element
    const int koff = KV8 ? it.kvh * D + c * (D / 4) + n * row_bytes       // + 16 i
                         : (it.kvh * D + 8 * c) * 2 + n * row_bytes;      // + 64 i
    const int voff = (it.kvh * D + EPL * n) * EB + 4 * c * row_bytes;     // + r * row_bytes
    const int addr_x32 = (lane ^ 32) * 4;

    auto load = [&](__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, Buf& buf) {
        if constexpr (KV8) {
#pragma unroll
            for (int i = 0; i < NQK / 2; ++i) buf.k[i] = load16<NT>(rk, koff + 16 * i);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (EPL == 8) buf.v[r] = load8<NT>(rv, voff + r * row_bytes);
                else buf.v[r] = load4<NT>(rv, voff + r * row_bytes);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NQK; ++i) buf.k[i] = load16<NT>(rk, koff + 64 * i);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (EPL == 8) buf.v[r] = load16<NT>(rv, voff + r * row_bytes);
                else buf.v[r] = load8<NT>(rv, voff + r * row_bytes);
            }
        }
    };

    // the K operand of MFMA i and the V rows, as 16-bit values of S
    auto k_operand = [&](const Buf& buf, int i) -> uint4 {
        if constexpr (KV8) {
            const uint32_t* w = reinterpret_cast<const uint32_t*>(buf.k) + 2 * i;
            const uint2 lo = fp8x4_to<S>(w[0]);
            const uint2 hi = fp8x4_to<S>(w[1]);
            return make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
            return buf.k[i];
        }
    };
    // dword q (16-bit elements 2q, 2q+1) of V row r, widened just before it is used
    auto v_word = [&](const Buf& buf, int r, int q) -> uint32_t {
        if constexpr (KV8) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(&buf.v[r])[q / 2];
            return (q & 1) ? S::template from_fp8x2<true>(w) : S::template from_fp8x2<false>(w);
        } else {
            return reinterpret_cast<const uint32_t*>(&buf.v[r])[q];
        }
    };

    // (!SPLIT) this wave's state into its LDS stage, then a fresh state.  kItem: the
    // result of partition p, written out from the stage so that every lane writes whole
    // lines (the accumulators sit in 16 of the 64 lanes, n < G).  kGroup: the state the
    // work-group merges.
    extern __shared__ float smem[];
    float* stage = smem + wave * G * (D + 4);     // [G][D], then (m, l) per head, 16-B aligned
    auto flush = [&](int p) {
        float lt = l + xor16(l);
        lt += xor32(lt, addr_x32);
        if (n < G) {
            float* dst = stage + n * D;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int e = 0; e < EPL; e += 4)
                    *reinterpret_cast<float4*>(dst + EPL * (4 * c + r) + e) =
                        make_float4(acc[e][r], acc[e + 1][r], acc[e + 2][r], acc[e + 3][r]);
            if (c == 0) *reinterpret_cast<float2*>(stage + G * D + 2 * n) = make_float2(m, lt);
        }
        // the LDS operations of one wave complete in order: the reads below see the writes
        if constexpr (MODE == kItem) store_partition<S, D>(a, it, G, p, stage, stage + G * D, lane);
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    };

    auto process = [&](int k, int valid, const Buf& buf) {
        f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NQK; ++i) s = S::mfma_k32(k_operand(buf, i), qv[i], s);
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
        // P^T operand as two 16-bit parts (rounded weights, then the rounded remainders):
        // both go through the matrix cores, so the weights enter the value product with
        // about 16 significand bits instead of the storage type's 8 or 11
        const uint2 p01 = split_pack2<S>(pr[0], pr[1]);
        const uint2 p23 = split_pack2<S>(pr[2], pr[3]);
        const uint2 pt = make_uint2(p01.x, p23.x);
        const uint2 ptl = make_uint2(p01.y, p23.y);
        // V^T operand of element e: (tok 4c, 4c+1 | 4c+2, 4c+3) at element EPL*n + e;
        // rows past the valid tokens were loaded as zeros
        // all rounded-part products first, then the remainders: the two products into one
        // accumulator are never back to back
        uint2 vev[EPL / 2], vod[EPL / 2];
#pragma unroll
        for (int q = 0; q < EPL / 2; ++q) {
            const uint32_t w0 = v_word(buf, 0, q);
            const uint32_t w1 = v_word(buf, 1, q);
            const uint32_t w2 = v_word(buf, 2, q);
            const uint32_t w3 = v_word(buf, 3, q);
            vev[q] = make_uint2(lo_halves(w0, w1), lo_halves(w2, w3));
            vod[q] = make_uint2(hi_halves(w0, w1), hi_halves(w2, w3));
            acc[2 * q] = S::mfma_k16(vev[q], pt, acc[2 * q]);
            acc[2 * q + 1] = S::mfma_k16(vod[q], pt, acc[2 * q + 1]);
        }
#pragma unroll
        for (int q = 0; q < EPL / 2; ++q) {
            acc[2 * q] = S::mfma_k16(vev[q], ptl, acc[2 * q]);
            acc[2 * q + 1] = S::mfma_k16(vod[q], ptl, acc[2 * q + 1]);
        }
        if constexpr (MODE == kItem) {     // last block of a partition: emit it
            const int j = walk.jb + k;
            if ((j + 1) % a.part_blocks == 0 || k + 1 == walk.nk) flush(j / a.part_blocks);
        }
    };

    if (a.new_k) {                                   // wave-uniform
        const int jl = (it.L - 1) / a.tile_tokens;   // the tile holding position L - 1
        bool mine = it.L > 0 && jl >= it.j0 && jl < it.j1;
        if constexpr (SPLIT) mine = mine && (jl - it.j0) % W == wave;
        if (mine) append_token<S, D, KV8>(a, it.b, it.kvh, it.L, lane);
    }

    // three register sets for every head size: with d = 64 a block's loads are small and
    // a wave's walk is latency-bound, so the third set pays (Qwen serving batch of 256:
    // 15.0 -> 13.9 us); a fourth does not
    if constexpr (PAIR) {
        PairWalk pw;
        pw.init_range(a, it, it.j0, it.j1, lane);
        const __amdgpu_buffer_rsrc_t lk = make_rsrc(a.k, a.layer_bytes);
        const __amdgpu_buffer_rsrc_t lv = make_rsrc(a.v, a.layer_bytes);
        // K row n of the tile: row n & 7 of block n >> 3; V rows 4c + r: block c >> 1
        const int krow = (n & 7) * row_bytes + (koff - n * row_bytes);
        const int vrow = 4 * (c & 1) * row_bytes + (voff - 4 * c * row_bytes);
        constexpr int kFar = 0x7FF80000;         // past any layer reached this way: loads zeros
        auto load_pair = [&](const PairLoc& loc, Buf& buf) {
            const bool k_first = n < 8;
            const int kb = k_first ? loc.off0 : loc.off1;
            const int kv = k_first ? loc.valid0 : loc.valid1;
            const int ko = (kb >= 0 && (n & 7) < kv) ? kb + krow : kFar;
            const bool v_first = c < 2;
            const int vb = v_first ? loc.off0 : loc.off1;
            const int vv = v_first ? loc.valid0 : loc.valid1;
            if constexpr (KV8) {
#pragma unroll
                for (int i = 0; i < NQK / 2; ++i) buf.k[i] = load16<NT>(lk, ko + 16 * i);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int vo = (vb >= 0 && 4 * (c & 1) + r < vv) ? vb + vrow + r * row_bytes : kFar;
                    if constexpr (EPL == 8) buf.v[r] = load8<NT>(lv, vo);
                    else buf.v[r] = load4<NT>(lv, vo);
                }
            } else {
#pragma unroll
                for (int i = 0; i < NQK; ++i) buf.k[i] = load16<NT>(lk, ko + 64 * i);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int vo = (vb >= 0 && 4 * (c & 1) + r < vv) ? vb + vrow + r * row_bytes : kFar;
                    if constexpr (EPL == 8) buf.v[r] = load16<NT>(lv, vo);
                    else buf.v[r] = load8<NT>(lv, vo);
                }
            }
        };
        walk_pairs3<Buf>(a, it, pw, load_pair, process);
    } else {
        walk_blocks3<Buf>(a, it, walk, row_bytes, load, process);
    }

    if constexpr (MODE == kGroup) {
        flush(it.p);
        __syncthreads();
        const int nchunks = (a.num_parts + per_item - 1) / per_item;
        const bool whole = chunk_id == 0 && it.nparts <= per_item;
        merge_slots_and_store<S, D>(a, it.b, it.kvh - wave % heads, heads,
                                    static_cast<int>(blockDim.x / 64) / heads, G, smem, chunk_id,
                                    nchunks, whole);
    }
    if constexpr (SPLIT) {
        // per-head totals: the four c-lanes of head n hold partial sums of l
        l += xor16(l);
        l += xor32(l, addr_x32);
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
        merge_waves_and_store<S, D>(a, it, G, sm_ml, sm_acc);
    }
}

// Waves of the group-plan kernel the GPU holds at once.
template <class S, int D, bool KV8>
int64_t group_target_waves() {
    static const int64_t waves =
        resident_waves(reinterpret_cast<const void*>(&pa_partition_mfma<S, D, kGroup, false, KV8>));
    return waves;
}

template <class S, int D, bool KV8>
hipError_t launch_t(int group, const DecodeArgs& a, hipStream_t stream) {
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads * a.num_parts;
    if (items <= 0) return hipSuccess;
    if (items > 0x7fffffff) return hipErrorInvalidValue;
    const size_t stage = static_cast<size_t>(group) * (D + 4) * sizeof(float);
    const Plan pl = make_plan(a, static_cast<int>(stage), true, group_target_waves<S, D, KV8>());
    if (pl.group_waves > 0) {
        // partials (if any) are per chunk: the reduce kernel sees chunks as partitions.
        // Work-groups keep launch order here: the XCDs then take neighbouring head
        // pairs of the same blocks, which measured faster than chunked renumbering.
        DecodeArgs g = a;
        g.xcd_chunk = 0;
        const int64_t wgs = static_cast<int64_t>(a.batch) * (a.num_kv_heads / pl.heads) * pl.chunks;
        // Whole sequences per work-group (one chunk, so no partial results in the
        // workspace) in many rounds of work-groups: the sequences go longest first, so
        // that the longest do not start last and run alone at the end.  The order sits at
        // the start of the workspace (at least B * Hq * 2 * (D + 2) floats whenever the
        // plan has more than one partition).  PAGEDKV_ORDER=0 keeps batch order, =1 orders
        // whenever the plan allows it.
        const char* eo = getenv("PAGEDKV_ORDER");
        const int64_t resident = group_target_waves<S, D, KV8>() / pl.group_waves;
        const bool may_order = pl.chunks == 1 && a.ws_acc != nullptr && a.batch > 1 &&
                               !a.keep_partials && a.pre_parts == 0;
        if (may_order && (eo ? eo[0] == '1' : wgs > 2 * resident)) {
            int32_t* order = reinterpret_cast<int32_t*>(a.ws_acc);
            hipLaunchKernelGGL(pa_length_order, dim3(1), dim3(kOrderThreads), 0, stream, a, order);
            g.order = order;
        }
        // 8-token blocks go two to a tile when one resource can reach the whole layer
        const bool pair = a.block_size == 8 && a.layer_bytes > 0 && !getenv_is0("PAGEDKV_PAIR");
        auto kernel = pair ? (a.stream_loads ? pa_partition_mfma<S, D, kGroup, true, KV8, true>
                                             : pa_partition_mfma<S, D, kGroup, false, KV8, true>)
                           : (a.stream_loads ? pa_partition_mfma<S, D, kGroup, true, KV8>
                                             : pa_partition_mfma<S, D, kGroup, false, KV8>);
        hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(wgs)), dim3(64 * pl.group_waves),
                           pl.group_waves * stage, stream, g, group, static_cast<int>(wgs),
                           pl.chunk, pl.ppw, pl.heads);
    } else if (split_items(items)) {
        hipLaunchKernelGGL((pa_partition_mfma<S, D, kSplit, false, KV8>), dim3(static_cast<unsigned>(items)),
                           dim3(64 * kWavesPerGroup), kWavesPerGroup * stage, stream, a, group,
                           static_cast<int>(items), 1, 1, 1);
    } else {
        static const int64_t slots =
            resident_waves(reinterpret_cast<const void*>(&pa_partition_mfma<S, D, kItem, false, KV8>));
        const int per = partitions_per_wave(items, slots, a.num_parts, a.part_blocks);
        const int64_t waves = static_cast<int64_t>(a.batch) * a.num_kv_heads * ceil_div(a.num_parts, per);
        const int64_t groups = (waves + kWavesPerGroup - 1) / kWavesPerGroup;
        auto kernel = a.stream_loads ? pa_partition_mfma<S, D, kItem, true, KV8>
                                     : pa_partition_mfma<S, D, kItem, false, KV8>;
        hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(groups)), dim3(64 * kWavesPerGroup),
                           kWavesPerGroup * stage, stream, a, group, static_cast<int>(waves), per,
                           1, 1);
    }
    return hipGetLastError();
}

// Calls F<S, D, KV8>::run(args...) for the dtypes and head size given at run time.
template <template <class, int, bool> class F, class... Args>
auto dispatch(int kv_dtype, int io_dtype, int head_dim, Args&&... args)
    -> decltype(F<F16, 64, false>::run(args...)) {
    const bool kv8 = kv_dtype == KV_DTYPE_FP8_E4M3;
    if (io_dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return kv8 ? F<F16, 64, true>::run(args...) : F<F16, 64, false>::run(args...);
        return kv8 ? F<F16, 128, true>::run(args...) : F<F16, 128, false>::run(args...);
    }
    if (head_dim == 64) return kv8 ? F<BF16, 64, true>::run(args...) : F<BF16, 64, false>::run(args...);
    return kv8 ? F<BF16, 128, true>::run(args...) : F<BF16, 128, false>::run(args...);
}

template <class S, int D, bool KV8> struct TargetWaves {
    static int64_t run() { return group_target_waves<S, D, KV8>(); }
};
template <class S, int D, bool KV8> struct Launch {
    static hipError_t run(int group, const DecodeArgs& a, hipStream_t stream) {
        return launch_t<S, D, KV8>(group, a, stream);
    }
};

}  // namespace

static Plan plan_mfma(int kv_dtype, int io_dtype, int group, int head_dim, const DecodeArgs& a) {
    const int stage = group * (head_dim + 4) * static_cast<int>(sizeof(float));
    const int64_t target = dispatch<TargetWaves>(kv_dtype, io_dtype, head_dim);
    return make_plan(a, stage, true, target);
}

int partition_chunk_mfma(int kv_dtype, int io_dtype, int group, int head_dim, const DecodeArgs& a) {
    return plan_mfma(kv_dtype, io_dtype, group, head_dim, a).chunk;
}

int group_waves_mfma(int kv_dtype, int io_dtype, int group, int head_dim, const DecodeArgs& a) {
    return plan_mfma(kv_dtype, io_dtype, group, head_dim, a).group_waves;
}

hipError_t launch_partitions_mfma(int kv_dtype, int io_dtype, int head_dim, int group,
                                  const DecodeArgs& a, hipStream_t stream) {
    if (group < 1 || group > 16) return hipErrorInvalidValue;
    if (head_dim != 64 && head_dim != 128) return hipErrorInvalidValue;
    if (io_dtype != KV_DTYPE_F16 && io_dtype != KV_DTYPE_BF16) return hipErrorInvalidValue;
    return dispatch<Launch>(kv_dtype, io_dtype, head_dim, group, a, stream);
}

}  // namespace pkv
