// Multi-token (prefill / chunked-prefill) paged attention on the matrix cores.
//
// A chunk of n new tokens of a sequence of length L sits at positions L - n .. L - 1;
// their keys and values are already in the pool.  Token i's query heads attend over
// positions [0, L - n + i] of the sequence, read through its block table: a prompt (or a
// chunk of one, cut to a step's token budget) processed in parallel, as "PagedAttention:
// Treating KV Memory Like Virtual Memory" ("Prefill is the other shape of the request")
// and "PagedAttention and Virtual Memory Management" (the prefill phase processes the
// prompt in parallel) describe it.
//
// Mapping.  The (token, query head) pairs of one (sequence, KV head) form n * G rows,
// head fastest; rows share the KV head's keys and values.  The decode kernel's matrix-
// core tile is reused with its 16 columns filled by 16 rows instead of G heads:
//   scores  S^T[16 keys][16 rows] = K[16 keys][D] . Q^T[D][16 rows]   (16x16x32 MFMA)
//   values  O^T[D][16 rows]      += V^T[D][16 keys] . P^T[16 keys][16 rows] (16x16x16)
// with a causal mask per column (key position <= the row's position) and a running max
// and sum per column.  Each wave owns NC column blocks (16 NC rows) so that every key /
// value tile it loads feeds NC products; a work-group of 4 waves covers 64 NC rows.
// A wave walks the key tiles from position 0 up to its last row's position; a column
// block whose rows all end before a tile skips that tile's products.  The keys of the
// 4 waves of a work-group are the same, so the second to fourth reads of a tile mostly
// hit the compute unit's cache.

#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "partition_common.h"

namespace pkv {
namespace {

template <bool KV8, int NQK, int EPL> struct PBuf;
template <int NQK, int EPL> struct PBuf<false, NQK, EPL> {
    uint4 k[NQK];
    typename std::conditional<EPL == 8, uint4, uint2>::type v[4];
};
template <int NQK, int EPL> struct PBuf<true, NQK, EPL> {
    uint4 k[NQK / 2];
    typename std::conditional<EPL == 8, uint2, uint32_t>::type v[4];
};

template <class S, int D, int NC, bool KV8>
__global__ __launch_bounds__(256) void pa_prefill_mfma(PrefillArgs pa) {
    const DecodeArgs& a = pa.a;
    constexpr int NQK = D / 32;
    constexpr int EPL = D / 16;
    using Buf = PBuf<KV8, NQK, EPL>;
    constexpr int kRowsPerWave = 16 * NC;
    constexpr int kRowsPerGroup = 4 * kRowsPerWave;

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;
    const int G = pa.group;

    // work-group -> (sequence, KV head, row tile); the heaviest row tiles (latest
    // positions, most keys) are numbered first
    const int rt = pa.row_tiles - 1 - static_cast<int>(blockIdx.x % pa.row_tiles);
    const int rest = static_cast<int>(blockIdx.x / pa.row_tiles);
    const int kvh = rest % a.num_kv_heads;
    const int b = rest / a.num_kv_heads;
    const int q0 = pa.qstart[b];
    const int nq = pa.qstart[b + 1] - q0;
    const int L = clamped_length(a, b);
    const int rows = nq * G;
    const int row_base = rt * kRowsPerGroup + wave * kRowsPerWave;
    if (rt * kRowsPerGroup >= rows) return;          // the whole work-group is past the chunk

    // this lane's column in each block: row -> (token, head), position, Q^T operand
    int qpos[NC];
    int tok[NC];
    uint4 qv[NC][NQK];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        const int r = row_base + cb * 16 + n;
        const int t = r / G;
        const int g = r - t * G;
        tok[cb] = t;
        qpos[cb] = (r < rows) ? L - nq + t : -1;     // -1: no such row / before position 0
        if (qpos[cb] < 0) qpos[cb] = -1;
        const size_t qrow = (static_cast<size_t>(q0 + t) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            const int e0 = KV8 ? c * (D / 4) + 8 * i : 8 * (4 * i + c);
            qv[cb][i] = qpos[cb] >= 0 ? *reinterpret_cast<const uint4*>(a.q + qrow + e0)
                                      : make_uint4(0, 0, 0, 0);
        }
    }
    // last position of each column block and of the wave (wave-uniform)
    int last[NC];
    int wave_last = -1;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        int x = qpos[cb];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) x = max(x, __shfl_xor(x, off));
        last[cb] = uniform(x);
        wave_last = max(wave_last, last[cb]);
    }
    __builtin_amdgcn_s_waitcnt(0);

    f32x4_t acc[NC][EPL];
    float m[NC], l[NC];
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        m[cb] = -INFINITY;
        l[cb] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[cb][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    const int row_bytes = a.row_bytes;
    constexpr int EB = KV8 ? 1 : 2;
    const int koff = KV8 ? kvh * D + c * (D / 4) + n * row_bytes : (kvh * D + 8 * c) * 2 + n * row_bytes;
    const int voff = (kvh * D + EPL * n) * EB + 4 * c * row_bytes;
    const int addr_x32 = (lane ^ 32) * 4;

    auto load = [&](__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, Buf& buf) {
        if constexpr (KV8) {
#pragma unroll
            for (int i = 0; i < NQK / 2; ++i) buf.k[i] = load16(rk, koff + 16 * i);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (EPL == 8) buf.v[r] = load8(rv, voff + r * row_bytes);
                else buf.v[r] = load4(rv, voff + r * row_bytes);
            }
        } else {
#pragma unroll
            for (int i = 0; i < NQK; ++i) buf.k[i] = load16(rk, koff + 64 * i);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (EPL == 8) buf.v[r] = load16(rv, voff + r * row_bytes);
                else buf.v[r] = load8(rv, voff + r * row_bytes);
            }
        }
    };
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
    auto v_word = [&](const Buf& buf, int r, int q) -> uint32_t {
        if constexpr (KV8) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(&buf.v[r])[q / 2];
            return (q & 1) ? S::template from_fp8x2<true>(w) : S::template from_fp8x2<false>(w);
        } else {
            return reinterpret_cast<const uint32_t*>(&buf.v[r])[q];
        }
    };

    Item it;
    it.b = b;
    it.kvh = kvh;
    it.L = L;
    BlockWalk walk;

    auto process = [&](int k, int valid, const Buf& buf) {
        const int tpos = (walk.jb + k) * a.tile_tokens;     // position of the tile's first key
        uint4 kop[NQK];
#pragma unroll
        for (int i = 0; i < NQK; ++i) kop[i] = k_operand(buf, i);
        uint2 pt[NC];
        bool live[NC];
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            live[cb] = last[cb] >= tpos;                     // wave-uniform
            pt[cb] = make_uint2(0, 0);
            if (!live[cb]) continue;
            f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < NQK; ++i) s = S::mfma_k32(kop[i], qv[cb][i], s);
            float sr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kr = 4 * c + r;
                sr[r] = (kr < valid && tpos + kr <= qpos[cb]) ? s[r] * a.scale_log2 : -INFINITY;
            }
            float mb = fmaxf(fmaxf(sr[0], sr[1]), fmaxf(sr[2], sr[3]));
            mb = fmaxf(mb, xor16(mb));
            mb = fmaxf(mb, xor32(mb, addr_x32));
            const float mn = fmaxf(m[cb], mb);
            const float mu = (mn == -INFINITY) ? 0.f : mn;
            const float alpha = fast_exp2(m[cb] - mu);
            float pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(sr[r] - mu);
            l[cb] = l[cb] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
            m[cb] = mn;
            if (__any(alpha != 1.f)) {
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[cb][e] *= alpha;
            }
            pt[cb] = make_uint2(S::pack2(pr[0], pr[1]), S::pack2(pr[2], pr[3]));
        }
        // V^T operand words, shared by the column blocks
#pragma unroll
        for (int q = 0; q < EPL / 2; ++q) {
            const uint32_t w0 = v_word(buf, 0, q);
            const uint32_t w1 = v_word(buf, 1, q);
            const uint32_t w2 = v_word(buf, 2, q);
            const uint32_t w3 = v_word(buf, 3, q);
            const uint2 even = make_uint2(lo_halves(w0, w1), lo_halves(w2, w3));
            const uint2 odd = make_uint2(hi_halves(w0, w1), hi_halves(w2, w3));
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                if (!live[cb]) continue;
                acc[cb][2 * q] = S::mfma_k16(even, pt[cb], acc[cb][2 * q]);
                acc[cb][2 * q + 1] = S::mfma_k16(odd, pt[cb], acc[cb][2 * q + 1]);
            }
        }
    };

    // tiles 0 .. (wave_last / T), in stretches of at most 256 (one table entry per lane
    // per tile held in four registers)
    const int ntiles = wave_last >= 0 ? wave_last / a.tile_tokens + 1 : 0;
    for (int j0 = 0; j0 < ntiles; j0 += kMaxTilesPerWave) {
        const int j1 = min(ntiles, j0 + kMaxTilesPerWave);
        walk.init_range(a, it, j0, j1, lane);
        __builtin_amdgcn_s_waitcnt(0);
        if constexpr (D == 128) walk_blocks3<Buf>(a, it, walk, row_bytes, load, process);
        else walk_blocks<Buf>(a, it, walk, row_bytes, load, process);
    }

    // normalise and write: lane (c, n) holds elements [c D/4, (c+1) D/4) of its row
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        float lt = l[cb] + xor16(l[cb]);
        lt += xor32(lt, addr_x32);
        const int r = row_base + cb * 16 + n;
        if (r >= rows) continue;
        const int t = tok[cb];
        const int g = r - t * G;
        const float inv = (qpos[cb] >= 0 && lt > 0.f) ? 1.f / lt : 0.f;
        uint16_t* dst = a.out + (static_cast<size_t>(q0 + t) * a.num_q_heads + kvh * G + g) * D + c * (D / 4);
        // acc[cb][e][rr] is element EPL (4c + rr) + e of the row
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            uint32_t w[EPL / 2];
#pragma unroll
            for (int e = 0; e < EPL; e += 2)
                w[e / 2] = S::pack2(acc[cb][e][rr] * inv, acc[cb][e + 1][rr] * inv);
            if constexpr (EPL == 8)
                *reinterpret_cast<uint4*>(dst + EPL * rr) = make_uint4(w[0], w[1], w[2], w[3]);
            else
                *reinterpret_cast<uint2*>(dst + EPL * rr) = make_uint2(w[0], w[1]);
        }
    }
}

template <class S, int D, bool KV8>
hipError_t launch_prefill_t(const PrefillArgs& pa, hipStream_t stream) {
    constexpr int NC = 2;
    const int64_t wgs = static_cast<int64_t>(pa.a.batch) * pa.a.num_kv_heads * pa.row_tiles;
    if (wgs <= 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    hipLaunchKernelGGL((pa_prefill_mfma<S, D, NC, KV8>), dim3(static_cast<unsigned>(wgs)), dim3(256),
                       0, stream, pa);
    return hipGetLastError();
}

}  // namespace

int prefill_rows_per_group() { return 4 * 16 * 2; }

hipError_t launch_prefill(int kv_dtype, int io_dtype, int head_dim, const PrefillArgs& pa,
                          hipStream_t stream) {
    const bool kv8 = kv_dtype == KV_DTYPE_FP8_E4M3;
    if (io_dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return kv8 ? launch_prefill_t<F16, 64, true>(pa, stream) : launch_prefill_t<F16, 64, false>(pa, stream);
        if (head_dim == 128) return kv8 ? launch_prefill_t<F16, 128, true>(pa, stream) : launch_prefill_t<F16, 128, false>(pa, stream);
    } else if (io_dtype == KV_DTYPE_BF16) {
        if (head_dim == 64) return kv8 ? launch_prefill_t<BF16, 64, true>(pa, stream) : launch_prefill_t<BF16, 64, false>(pa, stream);
        if (head_dim == 128) return kv8 ? launch_prefill_t<BF16, 128, true>(pa, stream) : launch_prefill_t<BF16, 128, false>(pa, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
