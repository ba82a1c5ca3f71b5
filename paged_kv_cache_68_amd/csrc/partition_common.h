// Pieces shared by the two partition kernels (VALU for single-head groups, MFMA for
// GQA groups): which (sequence, KV head, partition) a wave works on, how it finds its
// blocks through the block table, and how it walks them with a fixed number of loads
// in flight.
//
// Address translation follows "PagedAttention: Treating KV Memory Like Virtual Memory"
// ("How the kernel reads a block table": the tile at position i lives at
// block_table[i / B] * block stride + (i mod B) * slot stride) and section 4 of
// "PagedAttention and Virtual Memory Management" (Addr_K / Addr_V).  The block size B
// (8, 16, 32 or 64) is a power of two, so positions split into (block, slot) with a
// shift and a mask.  The kernels walk tiles of T = min(B, 16) tokens: a tile never
// straddles two blocks, a block holds B / T tiles, and the table is read once per tile,
// not per token.
#pragma once

#include <stdlib.h>

#include "device_common.h"

namespace pkv {

// One unit of work: partitions [p, p_end) of sequence b for KV head kvh, i.e. the
// sequence's tiles [j0, j1).  A wave that owns several consecutive partitions walks
// their tiles as one stream and emits one result per partition.
struct Item {
    int b, kvh;
    int p, p_end;
    int L;        // context length, clamped to the table width
    int nparts;   // partitions this sequence actually has
    int j0, j1;
};

// Tokens of sequence b that the table holds (its length less len_offset), clamped to
// [0, table width * B].
__device__ __forceinline__ int clamped_length(const DecodeArgs& a, int b) {
    const int L = a.lens[b] - a.len_offset;
    const int cap = a.max_blocks * a.block_size;
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Items are numbered with the KV head fastest, then the sequence, then the partition
// group: the 4 waves of a work-group take 4 KV heads of the same blocks.
__device__ __forceinline__ Item decode_item(const DecodeArgs& a, int item, int per_item) {
    Item it;
    it.kvh = item % a.num_kv_heads;
    const int rest = item / a.num_kv_heads;
    it.b = rest % a.batch;
    const int g = rest / a.batch;
    it.L = clamped_length(a, it.b);
    const int ntiles = (it.L + a.tile_tokens - 1) / a.tile_tokens;
    it.nparts = (ntiles + a.part_blocks - 1) / a.part_blocks;
    it.p = g * per_item;
    it.p_end = min(it.nparts, it.p + per_item);
    it.j0 = it.p * a.part_blocks;
    it.j1 = min(ntiles, it.p_end * a.part_blocks);
    return it;
}

// The tiles one wave visits: jb + js*k for k < nk.  The table entry of each tile's
// block sits one per lane in up to four VGPRs (at most 256 tiles) and is fetched once.
struct BlockWalk {
    int jb, js, nk;
    int tab[4];

    __device__ __forceinline__ void init(const DecodeArgs& a, const Item& it, int first, int step,
                                         int lane) {
        jb = it.j0 + first;
        js = step;
        nk = it.j1 > jb ? (it.j1 - jb + js - 1) / js : 0;
        const int32_t* trow = a.tables + static_cast<size_t>(it.b) * a.table_stride;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k = 64 * t + lane;
            tab[t] = (64 * t < nk && k < nk) ? trow[(jb + js * k) >> a.tiles_log2] : -1;
        }
    }

    // Tiles [j_begin, j_end) of the item's sequence, one after another.
    __device__ __forceinline__ void init_range(const DecodeArgs& a, const Item& it, int j_begin,
                                               int j_end, int lane) {
        jb = j_begin;
        js = 1;
        nk = j_end > jb ? j_end - jb : 0;
        const int32_t* trow = a.tables + static_cast<size_t>(it.b) * a.table_stride;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int k = 64 * t + lane;
            tab[t] = (64 * t < nk && k < nk) ? trow[(jb + k) >> a.tiles_log2] : -1;
        }
    }

    // k-th tile -> number of valid tokens and buffer resources over exactly those
    // token rows of K and V (empty past the last tile or for an out-of-range entry,
    // so loads there return zeros and read nothing).  Tile j is rows
    // [(j mod B/T) * T, ... + T) of block table[j / (B/T)].
    __device__ __forceinline__ int at(const DecodeArgs& a, const Item& it, int k, int row_bytes,
                                      __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv) const {
        int valid = 0;
        size_t off = 0;
        if (k < nk) {
            const int kk = k & 63;
            const int t = k < 64 ? __builtin_amdgcn_readlane(tab[0], kk)
                        : k < 128 ? __builtin_amdgcn_readlane(tab[1], kk)
                        : k < 192 ? __builtin_amdgcn_readlane(tab[2], kk)
                                  : __builtin_amdgcn_readlane(tab[3], kk);
            if (static_cast<unsigned>(t) < static_cast<unsigned>(a.num_blocks)) {
                const int j = jb + js * k;
                valid = min(a.tile_tokens, it.L - j * a.tile_tokens);
                const int row = (j & ((1 << a.tiles_log2) - 1)) * a.tile_tokens;
                off = (static_cast<size_t>(t) * a.block_size + row) * static_cast<size_t>(row_bytes);
            }
        }
        // everything here is wave-uniform; say so, or the resource would be rebuilt
        // lane by lane around every load
        valid = uniform(valid);
        const uint64_t uoff = (static_cast<uint64_t>(uniform(static_cast<int>(off >> 32))) << 32) |
                              static_cast<uint32_t>(uniform(static_cast<int>(off & 0xffffffffu)));
        rk = make_rsrc(a.k + uoff, valid * row_bytes);
        rv = make_rsrc(a.v + uoff, valid * row_bytes);
        return valid;
    }
};

// Run `process(k, valid, buf)` over the wave's blocks with two register sets used in
// turn.  Every iteration issues exactly one block's loads (an empty resource past the
// last block), so the wait before a block is computed always leaves the next block's
// loads in flight.
template <class Buf, class Load, class Process>
__device__ __forceinline__ void walk_blocks(const DecodeArgs& a, const Item& it, const BlockWalk& w,
                                            int row_bytes, Load load, Process process) {
    Buf ba, bb;
    __amdgpu_buffer_rsrc_t rk, rv;
    int valid_a = w.at(a, it, 0, row_bytes, rk, rv);
    load(rk, rv, ba);
    for (int k = 0; k < w.nk; k += 2) {
        const int valid_b = w.at(a, it, k + 1, row_bytes, rk, rv);
        load(rk, rv, bb);
        // keep the scheduler from sinking these loads into the computation below:
        // they must be issued before the wait for the current block's data
        __builtin_amdgcn_sched_barrier(0);
        process(k, valid_a, ba);
        if (k + 1 >= w.nk) break;
        valid_a = w.at(a, it, k + 2, row_bytes, rk, rv);
        load(rk, rv, ba);
        __builtin_amdgcn_sched_barrier(0);
        process(k + 1, valid_b, bb);
    }
}

// Same walk with three register sets: two blocks' loads stay in flight while one is
// computed.  For kernels whose register budget allows it at the same occupancy.
template <class Buf, class Load, class Process>
__device__ __forceinline__ void walk_blocks3(const DecodeArgs& a, const Item& it, const BlockWalk& w,
                                             int row_bytes, Load load, Process process) {
    Buf b0, b1, b2;
    __amdgpu_buffer_rsrc_t rk, rv;
    int v0 = w.at(a, it, 0, row_bytes, rk, rv);
    load(rk, rv, b0);
    int v1 = w.at(a, it, 1, row_bytes, rk, rv);
    load(rk, rv, b1);
    for (int k = 0; k < w.nk; k += 3) {
        const int v2 = w.at(a, it, k + 2, row_bytes, rk, rv);
        load(rk, rv, b2);
        __builtin_amdgcn_sched_barrier(0);
        process(k, v0, b0);
        if (k + 1 >= w.nk) break;
        v0 = w.at(a, it, k + 3, row_bytes, rk, rv);
        load(rk, rv, b0);
        __builtin_amdgcn_sched_barrier(0);
        process(k + 1, v1, b1);
        if (k + 2 >= w.nk) break;
        v1 = w.at(a, it, k + 4, row_bytes, rk, rv);
        load(rk, rv, b1);
        __builtin_amdgcn_sched_barrier(0);
        process(k + 2, v2, b2);
    }
}

// Partial results live in the workspace as [B][Hkv][P][G] rows (D floats of
// accumulator, 2 floats of running max / sum): the G heads of one item are one
// contiguous stretch, written with full, coalesced lines.
__device__ __forceinline__ size_t part_row(const DecodeArgs& a, int b, int kvh, int p, int G) {
    return ((static_cast<size_t>(b) * a.num_kv_heads + kvh) * a.num_parts + p) * G;
}

// A shared prefix handled elsewhere (pre_parts > 0) leaves, per query row (b * Hq + h),
// pre_parts partial results: int16 accumulators with a per-result scale, and (m, l).
// These fold results [s0, s1) of row `row`, elements [dd0, dd0 + 8), into the running
// state (Mt, L, acc) with the cross-block rule of "PagedAttention and Virtual Memory
// Management" section 4, in ascending order, eight at a time (their loads all in flight).
template <int D>
__device__ __forceinline__ void fold_prefix8(const DecodeArgs& a, size_t row, int dd0, int s0, int s1,
                                             float& Mt, float& L, float (&acc)[8]) {
    constexpr int U = 8;
    const int np = a.pre_parts;
    const float4* ml = reinterpret_cast<const float4*>(a.pre_ml) + row * np;
    const int16_t* q = a.pre_acc + row * np * D + dd0;
    for (int sb = s0; sb < s1; sb += U) {
        float4 e[U];
        uint4 qq[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = sb + u < s1;
            e[u] = ok ? ml[sb + u] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
            qq[u] = ok ? *reinterpret_cast<const uint4*>(q + static_cast<size_t>(sb + u) * D)
                       : make_uint4(0, 0, 0, 0);
        }
        float cm = e[0].x;
#pragma unroll
        for (int u = 1; u < U; ++u) cm = fmaxf(cm, e[u].x);
        if (cm > Mt) {                           // (Mt = -inf: nothing kept yet, so nothing scaled)
            const float f = (Mt == -INFINITY) ? 0.f : fast_exp2(Mt - cm);
            L *= f;
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] *= f;
            Mt = cm;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = (e[u].x == -INFINITY) ? 0.f : fast_exp2(e[u].x - Mt);
            L += w * e[u].y;
            const float ws = w * e[u].z;
            const uint32_t qw[4] = {qq[u].x, qq[u].y, qq[u].z, qq[u].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                acc[2 * k] += ws * static_cast<float>(static_cast<int16_t>(qw[k] & 0xffffu));
                acc[2 * k + 1] += ws * static_cast<float>(static_cast<int16_t>(qw[k] >> 16));
            }
        }
    }
}

// Two running states combined with the same rule: (Mt, L, acc) absorbs (Mq, Lq, accq).
__device__ __forceinline__ void fold_state8(float& Mt, float& L, float (&acc)[8], float Mq, float Lq,
                                            const float* accq) {
    const float Mn = fmaxf(Mt, Mq);
    const float f1 = (Mt == -INFINITY) ? 0.f : fast_exp2(Mt - Mn);
    const float f2 = (Mq == -INFINITY) ? 0.f : fast_exp2(Mq - Mn);
    L = f1 * L + f2 * Lq;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f1 * acc[k] + f2 * accq[k];
    Mt = Mn;
}

// Elements [dd0, dd0 + 8) of output row `row` from a running state.
template <class S, int D>
__device__ __forceinline__ void write_state8(const DecodeArgs& a, size_t row, int dd0, float L,
                                             const float (&acc)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        w[k] = static_cast<uint32_t>(S::narrow(L > 0.f ? acc[2 * k] / L : 0.f)) |
               (static_cast<uint32_t>(S::narrow(L > 0.f ? acc[2 * k + 1] / L : 0.f)) << 16);
    *reinterpret_cast<uint4*>(a.out + row * D + dd0) = make_uint4(w[0], w[1], w[2], w[3]);
}

// The final output of elements [dd0, dd0 + 8) of row `row`: this sequence's own result
// (M, lsum, A) first, then every prefix result in ascending order.
template <class S, int D>
__device__ __forceinline__ void cascade_store8(const DecodeArgs& a, size_t row, int dd0, float M,
                                               float lsum, const float (&A)[8]) {
    float Mt = M, L = lsum;
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = A[k];
    fold_prefix8<D>(a, row, dd0, 0, a.pre_parts, Mt, L, acc);
    write_state8<S, D>(a, row, dd0, L, acc);
}

// One wave writes the result of partition p of its item from a staging area in LDS
// (st_acc[G][D] accumulators, st_ml[G][2] running max / sum): the final output if the
// sequence has a single partition (combined first with a shared prefix's partial results
// when pre_parts > 0), else the fp32 partials.  All 64 lanes take part, each with 16-byte
// accesses, so the global writes are whole contiguous lines.  `whole`: the state covers
// every partition of the sequence; kept as a partial result (keep_partials) it is the
// only one, at slot 0 of rows [B][Hkv][1][G].
template <class S, int D>
__device__ __forceinline__ void store_partition(const DecodeArgs& a, const Item& it, int G, int p,
                                                const float* st_acc, const float* st_ml, int lane,
                                                bool whole = false) {
    const int n = G * D;
    if (a.pre_parts > 0) {           // (a single partition: the whole suffix)
        const size_t row0 = static_cast<size_t>(it.b) * a.num_q_heads + it.kvh * G;
        for (int i = lane * 8; i < n; i += 512) {
            const int g = i / D;
            const float4 x0 = *reinterpret_cast<const float4*>(st_acc + i);
            const float4 x1 = *reinterpret_cast<const float4*>(st_acc + i + 4);
            const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            cascade_store8<S, D>(a, row0 + g, i - g * D, st_ml[2 * g], st_ml[2 * g + 1], v);
        }
    } else if (!a.keep_partials && (it.nparts == 1 || whole)) {
        uint16_t* o = a.out + (static_cast<size_t>(it.b) * a.num_q_heads + it.kvh * G) * D;
        for (int i = lane * 8; i < n; i += 512) {
            const float lg = st_ml[2 * (i / D) + 1];
            const float4 x0 = *reinterpret_cast<const float4*>(st_acc + i);
            const float4 x1 = *reinterpret_cast<const float4*>(st_acc + i + 4);
            const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = static_cast<uint32_t>(S::narrow(lg > 0.f ? v[2 * e] / lg : 0.f)) |
                       (static_cast<uint32_t>(S::narrow(lg > 0.f ? v[2 * e + 1] / lg : 0.f)) << 16);
            *reinterpret_cast<uint4*>(o + i) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    } else {
        const size_t row0 = whole ? (static_cast<size_t>(it.b) * a.num_kv_heads + it.kvh) * G
                                  : part_row(a, it.b, it.kvh, p, G);
        float* dst = a.ws_acc + row0 * D;
        for (int i = lane * 4; i < n; i += 256)
            *reinterpret_cast<float4*>(dst + i) = *reinterpret_cast<const float4*>(st_acc + i);
        if (lane < 2 * G) a.ws_ml[row0 * 2 + lane] = st_ml[lane];
    }
}

// Four waves that shared one item have left their (m, l) in sm_ml[W][G][2] and their
// accumulators in sm_acc[W][G][D] (dimension order); merge them with the cross-block
// rule and write the partition's result: the final output if the sequence has a single
// partition (combined first with a shared prefix's partial results when pre_parts > 0),
// else the fp32 partials (m, l, acc) for the reduce kernel.
template <class S, int D>
__device__ __forceinline__ void merge_waves_and_store(const DecodeArgs& a, const Item& it, int G,
                                                      float* sm_ml, float* sm_acc) {
    constexpr int W = kWavesPerGroup;
    const int h0 = it.kvh * G;
    if (a.pre_parts > 0) {
        // (a single partition: the whole suffix) E groups of 8 output elements; Q threads
        // per group each fold an equal, consecutive share of the prefix results (one batch
        // of loads each for up to 32 of them); the first thread of each group then takes
        // the suffix's own result, its share and the others' shares in ascending order
        // (exchanged through the accumulators' LDS area once every wave's has been read).
        // Every thread of the work-group takes part: the two barriers are uniform.
        const int E = G * D / 8;
        const int Q = min(4, max(1, static_cast<int>(blockDim.x) / E));
        const int t = threadIdx.x;
        const int e = t % E;
        const int qi = t / E;
        const bool active = qi < Q;
        const int g = (e * 8) / D;
        const int dd0 = e * 8 - g * D;
        const size_t row = static_cast<size_t>(it.b) * a.num_q_heads + h0 + g;
        const int per = (a.pre_parts + Q - 1) / Q;
        float Mq = -INFINITY, Lq = 0.f;
        float accq[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) accq[k] = 0.f;
        if (active)
            fold_prefix8<D>(a, row, dd0, min(a.pre_parts, qi * per), min(a.pre_parts, (qi + 1) * per),
                            Mq, Lq, accq);
        float M = -INFINITY, lsum = 0.f;
        float A[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) A[k] = 0.f;
        if (active && qi == 0) {
            M = sm_ml[g * 2];
#pragma unroll
            for (int w = 1; w < W; ++w) M = fmaxf(M, sm_ml[(w * G + g) * 2]);
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float f = (M == -INFINITY) ? 0.f : fast_exp2(sm_ml[(w * G + g) * 2] - M);
                lsum += f * sm_ml[(w * G + g) * 2 + 1];
#pragma unroll
                for (int k = 0; k < 8; ++k) A[k] += f * sm_acc[(w * G + g) * D + dd0 + k];
            }
        }
        __syncthreads();                         // every wave's accumulators have been read
        float* xs = sm_acc;                      // shares 1 .. Q-1: [Q-1][E][10] floats
        if (active && qi > 0) {
            float* x = xs + ((qi - 1) * E + e) * 10;
            x[0] = Mq;
            x[1] = Lq;
#pragma unroll
            for (int k = 0; k < 8; ++k) x[2 + k] = accq[k];
        }
        __syncthreads();
        if (active && qi == 0) {
            fold_state8(M, lsum, A, Mq, Lq, accq);
            for (int j = 1; j < Q; ++j) {
                const float* x = xs + ((j - 1) * E + e) * 10;
                fold_state8(M, lsum, A, x[0], x[1], x + 2);
            }
            write_state8<S, D>(a, row, dd0, lsum, A);
        }
        return;
    }
    const size_t out_row0 = (static_cast<size_t>(it.b) * a.num_q_heads + h0) * D;
    for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
        const int g = idx / D;
        const int dd = idx % D;
        float M = sm_ml[g * 2];
#pragma unroll
        for (int w = 1; w < W; ++w) M = fmaxf(M, sm_ml[(w * G + g) * 2]);
        float lsum = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = (M == -INFINITY) ? 0.f : fast_exp2(sm_ml[(w * G + g) * 2] - M);
            lsum += f * sm_ml[(w * G + g) * 2 + 1];
            A += f * sm_acc[(w * G + g) * D + dd];
        }
        if (it.nparts == 1 && !a.keep_partials) {
            a.out[out_row0 + idx] = S::narrow(lsum > 0.f ? A / lsum : 0.f);
        } else {
            const size_t row = part_row(a, it.b, it.kvh, it.p, G) + g;
            a.ws_acc[row * D + dd] = A;
            if (dd == 0) {
                a.ws_ml[row * 2 + 0] = M;
                a.ws_ml[row * 2 + 1] = lsum;
            }
        }
    }
}

// A work-group of `heads` KV heads x `slots` waves per head has left every wave's state
// in LDS: wave w = hh + heads * s at smem + w * G * (D + 4), holding [G][D] accumulators
// and then (m, l) per query head.  Combine the slots of each head, in ascending order,
// with the cross-block rule.  If chunk c is the whole sequence the result is final;
// otherwise it is chunk c's partial result (rows [B][Hkv][nchunks][G]) for the reduce
// kernel.  The heads' output rows are contiguous, so the loop writes one stretch.
template <class S, int D>
__device__ __forceinline__ void merge_slots_and_store(const DecodeArgs& a, int b, int kvh0, int heads,
                                                      int slots, int G, const float* smem, int c,
                                                      int nchunks, bool whole) {
    const int stride = G * (D + 4);
    const int per_head = G * D;
    const size_t out0 = (static_cast<size_t>(b) * a.num_q_heads + kvh0 * G) * D;
    for (int idx = threadIdx.x; idx < heads * per_head; idx += blockDim.x) {
        const int hh = idx / per_head;
        const int rem = idx - hh * per_head;
        const int g = rem / D;
        const int dd = rem - g * D;
        const float* st0 = smem + hh * stride;
        const int step = heads * stride;
        float M = -INFINITY;
        for (int s = 0; s < slots; ++s) M = fmaxf(M, st0[s * step + per_head + 2 * g]);
        float lsum = 0.f, A = 0.f;
        for (int s = 0; s < slots; ++s) {
            const float* st = st0 + s * step;
            const float f = (M == -INFINITY) ? 0.f : fast_exp2(st[per_head + 2 * g] - M);
            lsum += f * st[per_head + 2 * g + 1];
            A += f * st[rem];
        }
        if (whole && !a.keep_partials) {
            a.out[out0 + idx] = S::narrow(lsum > 0.f ? A / lsum : 0.f);
        } else {
            const size_t row =
                ((static_cast<size_t>(b) * a.num_kv_heads + kvh0 + hh) * nchunks + c) * G + g;
            a.ws_acc[row * D + dd] = A;
            if (dd == 0) {
                a.ws_ml[row * 2 + 0] = M;
                a.ws_ml[row * 2 + 1] = lsum;
            }
        }
    }
}

// Zero output for a sequence with no tokens (written once, by partition 0's item).  With
// keep_partials nothing: such a sequence has no partial results.  With a shared prefix
// handled elsewhere (pre_parts > 0), the prefix's partial results alone.
template <class S, int D>
__device__ __forceinline__ void store_empty(const DecodeArgs& a, const Item& it, int G, int t0, int nt) {
    if (it.p != 0) return;
    if (a.pre_parts > 0) {
        const size_t row0 = static_cast<size_t>(it.b) * a.num_q_heads + it.kvh * G;
        const float none[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int i = t0 * 8; i < G * D; i += nt * 8)
            cascade_store8<S, D>(a, row0 + i / D, i % D, -INFINITY, 0.f, none);
        return;
    }
    if (a.keep_partials) return;
    const size_t out_row0 = (static_cast<size_t>(it.b) * a.num_q_heads + it.kvh * G) * D;
    for (int i = t0; i < G * D; i += nt) a.out[out_row0 + i] = 0;
}

// Work-groups per XCD chunk in the launch renumbering (see xcd_chunked).
constexpr int kXcdChunk = 16;

// Choose between one wave per item and four waves sharing an item.  PAGEDKV_SPLIT=0/1
// forces one of them (used by the tests to cover both on small inputs).
inline bool split_items(int64_t items) {
    const char* env = getenv("PAGEDKV_SPLIT");
    if (env && (env[0] == '0' || env[0] == '1')) return env[0] == '1';
    return items < 4096;
}

// Waves of `kernel` (256-thread work-groups) the GPU holds at once.
inline int64_t resident_waves(const void* kernel) {
    int dev = 0, cus = 0, blocks = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, 64 * kWavesPerGroup, 0) !=
            hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return static_cast<int64_t>(cus) * blocks * kWavesPerGroup;
}

// Partitions per wave when waves own whole items: enough waves for about two rounds
// of the GPU's resident waves (`slots`), at most 256 blocks of table per wave.
inline int partitions_per_wave(int64_t items, int64_t slots, int num_parts, int part_tiles) {
    const char* env = getenv("PAGEDKV_PARTS_PER_WAVE");     // override, for the tests
    int64_t per = env ? atoi(env) : (slots > 0 ? items / (2 * slots) : 1);
    const int64_t cap = kMaxTilesPerWave / part_tiles;
    if (per > num_parts) per = num_parts;
    if (per > cap) per = cap;
    return per < 1 ? 1 : static_cast<int>(per);
}

// Compute units of the current device (0 if the query fails).
inline int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return cus;
}

// True when the variable is set to a value starting with '0' (a tuning switch turned off).
inline bool getenv_is0(const char* name) {
    const char* e = getenv(name);
    return e && e[0] == '0';
}

inline int env_int(const char* name, int fallback) {
    const char* e = getenv(name);
    return (e && atoi(e) > 0) ? atoi(e) : fallback;
}

// How the partition kernel covers the batch.  In the group plan a work-group owns
// `heads` consecutive KV heads of one sequence and `slots` waves per head; each wave
// walks `ppw` consecutive partitions of its head as one stream (the cross-block rule
// applied block by block), and the work-group merges its waves in LDS.  One work-group
// covers `chunk` = slots * ppw partitions of a head; with chunks = ceil(P / chunk) > 1
// the reduce kernel combines the chunks' partial results like partitions of
// chunk * part_blocks blocks.  Outside the group plan chunk = 1.
struct Plan {
    int group_waves;   // > 0: group plan with work-groups of this many waves
    int heads;
    int slots;
    int ppw;
    int chunk;
    int chunks;
};

// Choice of the group plan (MFMA kernel, enough work, more than one partition).  The
// waves of all work-groups together about fill the GPU once (`target_waves`); each
// walks at most 256 tiles (its table entries sit in four registers) and every wave's
// LDS stage stays within 64 KiB.
//  * Long sequences streamed from HBM (at least two waves per (sequence, KV head), and
//    more bytes than the last-level cache holds, see streamed): work-groups of 8
//    waves spanning as many KV heads as make about 1 KiB of each token row (4 heads of
//    128 bf16 / fp16 values, 8 of FP8), i.e. whole contiguous stretches of the row
//    instead of separate 128- or 256-byte pieces fetched by unrelated work-groups; the
//    remaining waves of a head are its slots, each walking an equal share of the
//    partitions.  A sequence is cut into as many chunks as give one work-group per
//    compute unit; the reduce kernel combines the chunks' partial results (about 2 KB
//    per (sequence, head) and chunk).  Measured
//    on 64 x 8,192 tokens (Llama-3-8B heads): 329 -> 321 us for bf16 and 190 -> 176 us
//    for FP8 against two heads per work-group with the whole sequence in one.
//  * Otherwise (many short items, or a working set the cache serves, where the extra
//    chunks cost): as many KV heads as make 512 contiguous bytes of each token row (2
//    heads of 128 16-bit values, 4 of 128 FP8 codes: 2,641 against 2,892 us per step on
//    512 FP8 sequences of U[1, 4096] tokens with 64 heads, against 2) while that still
//    leaves a work-group per compute unit, enough chunks for one work-group per compute
//    unit, and slots to fill the GPU.
// PAGEDKV_GROUP=0 disables the plan; PAGEDKV_GROUP_HEADS / _SLOTS / _PPW override it.
inline Plan make_plan(const DecodeArgs& a, int stage_bytes, bool group_capable,
                      int64_t target_waves) {
    Plan pl{0, 1, 1, 1, 1, a.num_parts};
    const int P = a.num_parts;
    const int64_t items = static_cast<int64_t>(a.batch) * a.num_kv_heads * P;
    const char* env = getenv("PAGEDKV_GROUP");
    const bool allowed = group_capable && !(env && env[0] == '0') && !split_items(items);
    if (!allowed || P < 2) return pl;
    const int64_t seqheads = static_cast<int64_t>(a.batch) * a.num_kv_heads;
    const int64_t cus = device_cus() > 0 ? device_cus() : 256;
    if (target_waves <= 0) target_waves = 8 * cus;

    const int64_t per_head = target_waves / seqheads;     // waves per (sequence, KV head)
    int heads, chunk, ppw;
    int64_t slots;
    if (per_head >= 2 && a.streamed) {
        const int head_bytes = a.row_bytes / a.num_kv_heads;
        heads = 1;
        while (heads * 2 <= 8 && a.num_kv_heads % (heads * 2) == 0 && heads * 2 * head_bytes <= 1024)
            heads *= 2;
        // one work-group per compute unit: chunks of the sequence as needed
        const int64_t groups = seqheads / heads;
        int64_t chunks = (cus + groups - 1) / groups;
        if (chunks > P) chunks = P;
        chunk = static_cast<int>((P + chunks - 1) / chunks);
        slots = 8 / heads;
        while (slots > 1 && heads * slots * stage_bytes > 64 * 1024) --slots;
        if (slots > chunk) slots = chunk;
        ppw = (chunk + static_cast<int>(slots) - 1) / static_cast<int>(slots);
    } else {
        // as many heads as make 512 contiguous bytes of each token row (2 of 128 16-bit
        // values, 4 of 128 FP8 codes) while leaving a work-group per compute unit
        const int head_bytes = a.row_bytes / a.num_kv_heads;
        heads = 1;
        while (a.num_kv_heads % (heads * 2) == 0 && heads * 2 * head_bytes <= 512 &&
               seqheads / (heads * 2) >= cus)
            heads *= 2;
        int64_t chunks = (cus + seqheads / heads - 1) / (seqheads / heads);
        if (chunks > P) chunks = P;
        chunk = static_cast<int>((P + chunks - 1) / chunks);
        slots = (target_waves + seqheads * chunks - 1) / (seqheads * chunks);
        if (slots > 8 / heads) slots = 8 / heads;
        if (slots > chunk) slots = chunk;
        ppw = (chunk + static_cast<int>(slots) - 1) / static_cast<int>(slots);
    }

    // overrides: the work-group shape is then taken as given (within the limits below)
    const bool forced = getenv("PAGEDKV_GROUP_HEADS") || getenv("PAGEDKV_GROUP_SLOTS") ||
                        getenv("PAGEDKV_GROUP_PPW");
    if (forced) {
        heads = env_int("PAGEDKV_GROUP_HEADS", heads);
        slots = env_int("PAGEDKV_GROUP_SLOTS", static_cast<int>(slots));
        ppw = env_int("PAGEDKV_GROUP_PPW", ppw);
        chunk = P;
    }
    if (heads > 8 || a.num_kv_heads % heads != 0) heads = 1;
    if (slots > 8 / heads) slots = 8 / heads;
    while (slots > 1 && heads * slots * stage_bytes > 64 * 1024) --slots;
    if (slots < 1) slots = 1;
    const int max_ppw = kMaxTilesPerWave / a.part_blocks;
    if (ppw > max_ppw) ppw = max_ppw;
    if (slots * ppw < chunk) chunk = static_cast<int>(slots) * ppw;
    slots = (chunk + ppw - 1) / ppw;        // no wave without a partition
    pl.heads = heads;
    pl.slots = static_cast<int>(slots);
    pl.ppw = ppw;
    pl.group_waves = heads * pl.slots;
    pl.chunk = chunk;
    pl.chunks = (P + chunk - 1) / chunk;
    return pl;
}

}  // namespace pkv
