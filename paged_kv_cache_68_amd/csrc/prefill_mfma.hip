// Multi-token (prefill / chunked-prefill) paged attention on the matrix cores.
//
// A chunk of n new tokens of a sequence of length L sits at positions L - n .. L - 1;
// their keys and values are already in the pool.  Token i's query heads attend over
// positions [0, L - n + i] of the sequence, read through its block table: a prompt (or a
// chunk of one, cut to a step's token budget) processed in parallel, as "PagedAttention:
// Treating KV Memory Like Virtual Memory", section "What the allocator actually sees"
// (besides one-token decode steps, a request also arrives as a whole prompt, or pieces
// of one sized to the step's token budget), and "PagedAttention and Virtual Memory
// Management" (the prefill phase processes the prompt in parallel) describe it.
//
// Mapping.  The (token, query head) pairs of one (sequence, KV head) form n * G rows,
// head fastest; rows share the KV head's keys and values.  A work-group of W waves owns
// 32 W consecutive rows, each wave two column blocks of 16 rows, and walks the keys
// from position 0 to its last row's position in stages of 64 keys (one barrier per
// stage; fewer barriers keep the waves from falling into step with each other), each
// computed as two runs of 32:
//  * the work-group's threads fetch a stage's keys and values through the block table
//    (one 16-byte LDS chunk of 8 values per thread and tensor at a time; E4M3 codes are
//    widened here, once per work-group) into one of two LDS buffers, while the waves
//    compute on the other;
//  * scores  S^T[16 keys][16 rows] = K . Q^T     (16x16x32 MFMA, two per run and k-chunk)
//  * values  O^T[16 d][16 rows]   += V^T . P^T   (16x16x32 MFMA over the run's 32 keys)
//    the P^T operand is the score tile's own register layout (key slot 8c + j of the
//    product is key 4c + j of the first 16 and 16 + 4c + j - 4 of the second), and the
//    V^T operand takes the same slots from LDS transpose reads (ds_read_b64_tr_b16);
//  * online softmax per column (base 2) with a lazy rescale: the running maximum is
//    raised only when a score passes it by more than 2^8, so the weights stay below 256
//    and the accumulator is rescaled rarely; each lane checks its own scores and the
//    column maximum is formed only then; the weight sums come from one more MFMA with an
//    all-ones operand; a run that lies wholly before every row of a wave needs no
//    causal mask.
// Keys past the sequence's length (and table entries outside the pool) are staged as
// zeros, so masked weights never meet stale memory.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "partition_common.h"

namespace pkv {
namespace {

// Row-pair lane swaps (gfx950 v_permlane16_swap / v_permlane32_swap) of one value with
// itself: a = the value of the even row (or the lower half), b = that of the odd row (or
// the upper half), in every lane of the pair.  The second operand is passed through an
// empty asm statement so that the compiler cannot treat the two operands as one value:
// it would otherwise fold the second result into the first.
struct pair_f {
    float a, b;
};
__device__ __forceinline__ pair_f swap16(float x) {
    uint32_t y = __builtin_bit_cast(uint32_t, x);
    asm volatile("" : "+v"(y));
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), y, false, false);
    return {__builtin_bit_cast(float, static_cast<uint32_t>(r[0])), __builtin_bit_cast(float, static_cast<uint32_t>(r[1]))};
}
__device__ __forceinline__ pair_f swap32(float x) {
    uint32_t y = __builtin_bit_cast(uint32_t, x);
    asm volatile("" : "+v"(y));
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), y, false, false);
    return {__builtin_bit_cast(float, static_cast<uint32_t>(r[0])), __builtin_bit_cast(float, static_cast<uint32_t>(r[1]))};
}

constexpr int kPfRowsPerWave = 32;  // two 16-row column blocks

constexpr int kPfRuns = 2;          // 32-key runs per LDS stage (one barrier per stage)

// A split launch gives each row tile its own number of key-range splits: at most the
// planned count, and no more than leave every split at least this many 64-key stages.
// A tile with one split writes its rows' output itself and needs no merge.
constexpr int kMinSplitStages = 4;
__device__ __forceinline__ int tile_splits(int planned, int nstages) {
    return min(planned, max(1, nstages / kMinSplitStages));
}

// SPLIT: pa.splits work-groups share each row tile's key stages, each taking an equal
// run of them and writing its rows' unnormalised partial results (acc, m, l) for
// pa_prefill_merge to combine.
// DENSE (with SPLIT): the shared prefix of a decode batch.  The batch's queries are the
// rows of one "sequence" (token t = sequence t, all num_tokens of them), the keys are
// positions [0, dense_len) of table row 0, and row t's causal limit is its own length:
// it sees keys [0, min(lens[t], dense_len)).  The partial results cover the prefix only;
// the suffix of each sequence is walked by the decode kernels, which combine the two
// (or leave theirs for the cascade reduce).
template <class S, int D, int W, bool KV8, bool SPLIT, bool DENSE = false>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2))) void pa_prefill_mfma(PrefillArgs pa) {
    static_assert(!DENSE || SPLIT, "the dense form writes partial results");
    const DecodeArgs& a = pa.a;
    constexpr int NC = 2;
    constexpr int KT = 32 * kPfRuns;             // keys per LDS stage
    constexpr int NQK = D / 32;                  // k-chunks of the score product
    constexpr int DB = D / 16;                   // 16-row d-blocks of the value product
    // LDS bytes per staged key and value row: the padding spreads the rows over the banks
    // for the key reads (16 rows, one 16-byte chunk each) and the value transpose reads
    // (8 rows, 32 bytes each, per half wave).  Measured on the kernel's own address
    // patterns: with 32 bytes both read at the linear rate; 16 bytes cut the key reads to
    // 58% of it, and unpadded value rows cut the transposing reads to a sixth
    constexpr int ROWB_K = D * 2 + 32;
    constexpr int ROWB_V = D * 2 + 32;
    constexpr int CPR = D / 8;                   // 16-byte LDS chunks per key row
    constexpr int CHUNKS = KT * CPR;             // chunks per tensor and stage
    constexpr int THREADS = 64 * W;
    constexpr int PER_T = (CHUNKS + THREADS - 1) / THREADS;
    constexpr int EB = KV8 ? 1 : 2;              // bytes per stored element
    constexpr int STAGE_K = KT * ROWB_K;
    constexpr int STAGE_V = KT * ROWB_V;
    using Raw = typename std::conditional<KV8, uint2, uint4>::type;
    constexpr bool kSplitWeights = std::is_same<S, BF16>::value;

    __shared__ __align__(16) uint8_t lds_k[2][STAGE_K];
    __shared__ __align__(16) uint8_t lds_v[2][STAGE_V];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;
    const int G = pa.group;

    // work-group -> (sequence, KV head, row tile[, split]); the heaviest row tiles (latest
    // positions, most keys) are numbered first.  The launch goes round the 8 XCDs one
    // work-group at a time; renumbered, the work-groups of one (sequence, KV head), which
    // all stage the same keys and values, run on one XCD and meet in its L2 (6% faster
    // on the chunked-prefill step; not for the dense form, whose work-groups of a KV head
    // each stage a different range of keys)
    const int bid = DENSE ? static_cast<int>(blockIdx.x)
                          : xcd_chunked(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x),
                                        pa.row_tiles * (SPLIT ? pa.splits : 1));
    const int split = SPLIT ? bid % pa.splits : 0;
    const int tile_id = SPLIT ? bid / pa.splits : bid;
    const int rt = pa.row_tiles - 1 - tile_id % pa.row_tiles;
    const int rest = tile_id / pa.row_tiles;
    const int kvh = rest % a.num_kv_heads;
    const int b = DENSE ? 0 : rest / a.num_kv_heads;
    const int q0 = DENSE ? 0 : pa.qstart[b];
    const int nq = DENSE ? pa.num_tokens : pa.qstart[b + 1] - q0;
    const int L = DENSE ? pa.dense_len : clamped_length(a, b);
    const int rows = nq * G;
    const int group_row0 = rt * kPfRowsPerWave * W;
    if (group_row0 >= rows) return;              // the whole work-group is past the chunk
    const int row_base = group_row0 + wave * kPfRowsPerWave;
    // a negative scale is applied as a positive one to the negated query (exact), so that
    // the running maximum of the raw scores is that of the scaled ones (a zero scale runs
    // as 1e-30: every weight is then exactly 1, as it should be, and masked scores stay
    // -inf instead of becoming 0 * inf)
    const float sl2 = fmaxf(fabsf(a.scale_log2), 1e-30f);
    const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;

    // ---- staging: global (through the table) -> registers -> LDS.  Thread chunk u is
    // key (tid + u THREADS) / CPR of the stage, 8 values at part (tid + u THREADS) % CPR.
    const int* table = a.tables + static_cast<size_t>(b) * a.table_stride;
    const int bshift = __builtin_ctz(a.block_size);
    const uint32_t block_bytes = static_cast<uint32_t>(a.block_size * a.row_bytes);
    Raw rk[PER_T], rv[PER_T];
    int tb[PER_T];                               // table entries of the stage being fetched
    const __amdgpu_buffer_rsrc_t rsrc_k = make_rsrc(a.k, pa.buffer_bytes);
    const __amdgpu_buffer_rsrc_t rsrc_v = make_rsrc(a.v, pa.buffer_bytes);

    auto fetch_table = [&](int j) {
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
            const int q = tid + u * THREADS;
            const int pos = j * KT + q / CPR;
            tb[u] = (q < CHUNKS && pos < L) ? table[pos >> bshift] : -1;
        }
    };
    auto fetch = [&](int j) {
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
            const int q = tid + u * THREADS;
            const int pos = j * KT + q / CPR;
            const int blk = tb[u];
            const bool ok = q < CHUNKS && static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks);
            const uint32_t inner = static_cast<uint32_t>((pos & (a.block_size - 1)) * a.row_bytes +
                                                         (kvh * D + (q % CPR) * 8) * EB);
            if (pa.buffer_bytes > 0) {
                // an entry outside the pool (or past the length) reads past the buffer's
                // end, which returns zeros
                const uint32_t off = ok ? static_cast<uint32_t>(blk) * block_bytes + inner : 0x80000000u;
                if constexpr (KV8) {
                    rk[u] = load8(rsrc_k, static_cast<int>(off));
                    rv[u] = load8(rsrc_v, static_cast<int>(off));
                } else {
                    rk[u] = load16(rsrc_k, static_cast<int>(off));
                    rv[u] = load16(rsrc_v, static_cast<int>(off));
                }
            } else {
                // an entry outside the pool (or past the length) reads block 0 and stages zeros
                const size_t off = static_cast<size_t>(ok ? static_cast<uint32_t>(blk) : 0u) * block_bytes + inner;
                const Raw xk = *reinterpret_cast<const Raw*>(a.k + off);
                const Raw xv = *reinterpret_cast<const Raw*>(a.v + off);
                rk[u] = ok ? xk : Raw{};
                rv[u] = ok ? xv : Raw{};
            }
        }
    };
    auto widen = [&](const Raw& x) -> uint4 {
        if constexpr (KV8) {
            const uint2 lo = fp8x4_to<S>(x.x);
            const uint2 hi = fp8x4_to<S>(x.y);
            return make_uint4(lo.x, lo.y, hi.x, hi.y);
        } else {
            return x;
        }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
        for (int u = 0; u < PER_T; ++u) {
            const int q = tid + u * THREADS;
            if (q < CHUNKS) {
                *reinterpret_cast<uint4*>(&lds_k[buf][(q / CPR) * ROWB_K + (q % CPR) * 16]) = widen(rk[u]);
                *reinterpret_cast<uint4*>(&lds_v[buf][(q / CPR) * ROWB_V + (q % CPR) * 16]) = widen(rv[u]);
            }
        }
    };

    // dense: the key range is known from the arguments alone, so the first stage's table
    // entries and rows are requested before anything else (ahead of the queries and the
    // lengths, which only the masks need)
    int j_lo = 0, j_hi = 0;
    if constexpr (DENSE) {
        const int ns = (L + KT - 1) / KT;
        const int per = (ns + pa.splits - 1) / pa.splits;
        j_lo = min(ns, split * per);
        j_hi = min(ns, j_lo + per);
        if (j_lo < j_hi) {
            fetch_table(j_lo);
            fetch(j_lo);
        }
    }

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
        if constexpr (DENSE) {
            qpos[cb] = (r < rows) ? min(max(a.lens[t], 0), L) - 1 : -1;
        } else {
            qpos[cb] = (r < rows) ? L - nq + t : -1;     // -1: no such row / before position 0
            if (qpos[cb] < 0) qpos[cb] = -1;
        }
        const size_t qrow = (static_cast<size_t>(q0 + t) * a.num_q_heads + kvh * G + g) * D;
#pragma unroll
        for (int i = 0; i < NQK; ++i) {
            qv[cb][i] = qpos[cb] >= 0 ? *reinterpret_cast<const uint4*>(a.q + qrow + 32 * i + 8 * c)
                                      : make_uint4(0, 0, 0, 0);
            qv[cb][i].x ^= qsign;
            qv[cb][i].y ^= qsign;
            qv[cb][i].z ^= qsign;
            qv[cb][i].w ^= qsign;
        }
    }
    // first and last position of each column block (wave-uniform): rows are in token
    // order, so the block's first row has its smallest position (dense: any order, so
    // the smallest is searched for)
    int last[NC];
    int first[NC];
    int wave_last = -1;
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        int x = qpos[cb];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) x = max(x, __shfl_xor(x, off));
        last[cb] = uniform(x);
        wave_last = max(wave_last, last[cb]);
        const int r0 = row_base + cb * 16;
        if constexpr (DENSE) {
            int y = qpos[cb];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) y = min(y, __shfl_xor(y, off));
            first[cb] = uniform(y);
        } else {
            first[cb] = r0 < rows ? L - nq + r0 / G : -1;
        }
    }
    // the work-group's last position: its last row's (dense: the prefix's last key)
    const int group_rows_end = min(rows, group_row0 + kPfRowsPerWave * W);
    const int group_last = DENSE ? L - 1 : L - nq + (group_rows_end - 1) / G;
    const int nstages = group_last >= 0 ? group_last / KT + 1 : 0;
    const int wave_stages = wave_last >= 0 ? wave_last / KT + 1 : 0;

    f32x4_t acc[NC][DB];
    f32x4_t lacc[NC];                            // running sums of the weights (4 equal rows)
    float m[NC];
    const uint32_t one2 = S::pack2(1.f, 1.f);
    const uint4 ones = make_uint4(one2, one2, one2, one2);
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        m[cb] = -INFINITY;
        lacc[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < DB; ++e) acc[cb][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // ---- one run of 32 keys for this wave.  Both column blocks always run: a block
    // whose rows all precede the run gets only masked scores, zero weights and no
    // change, and the straight-line code lets the LDS reads run ahead of the products.
    // V^T operands come from LDS transpose reads: in each 16-lane group, source lane s
    // reads 4 values of key slot s / 4 at d offset 4 (s % 4), and lane n receives the
    // 4 slots' values of d row n.
    const int tr_key = 4 * c + (n >> 2);         // key of this lane's transpose source slot
    const int tr_d = 4 * (n & 3);
    auto max_across_c = [](float x) {            // over the 4 lanes of a column (lane ^ 16, ^ 32)
        const pair_f r = swap16(x);
        x = __builtin_fmaxf(r.a, r.b);
        const pair_f t = swap32(x);
        return __builtin_fmaxf(t.a, t.b);
    };
    auto compute_half = [&](int tpos, const uint8_t* kl, const uint8_t* vl) {
        uint4 kop[2][NQK];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < NQK; ++i)
                kop[st][i] = *reinterpret_cast<const uint4*>(kl + (st * 16 + n) * ROWB_K + (32 * i + 8 * c) * 2);
        // V^T operand of d-block e: slots 8c .. 8c + 3 are keys 4c .. 4c + 3, slots
        // 8c + 4 .. 8c + 7 keys 16 + 4c .. 16 + 4c + 3
        uint4 vop[DB];
#pragma unroll
        for (int e = 0; e < DB; ++e) {
            typedef short v4i16 __attribute__((ext_vector_type(4)));
            typedef v4i16 __attribute__((address_space(3))) lds_v4i16;
            const uint8_t* p0 = vl + tr_key * ROWB_V + (16 * e + tr_d) * 2;
            const uint8_t* p1 = p0 + 16 * ROWB_V;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(__attribute__((address_space(3))) const uint8_t*)(p0));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4i16*)(__attribute__((address_space(3))) const uint8_t*)(p1));
            const uint2 l2 = __builtin_bit_cast(uint2, lo);
            const uint2 h2 = __builtin_bit_cast(uint2, hi);
            vop[e] = make_uint4(l2.x, l2.y, h2.x, h2.y);
        }
        f32x4_t sc[NC][2];
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < NQK; ++i) x = S::mfma_k32(kop[st][i], qv[cb][i], x);
                sc[cb][st] = x;
            }
        uint4 pop[NC], pol[NC];                  // weights: rounded parts, remainders
        float sv[NC][8];
#pragma unroll
        for (int cb = 0; cb < NC; ++cb)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
                for (int r = 0; r < 4; ++r) sv[cb][4 * st + r] = sc[cb][st][r];
        // The mask and the rare rescale are one branch each for both column blocks, so that
        // the weights and value products of both blocks form one stretch of code for the
        // scheduler (8% faster on the chunked-prefill step than a branch per block).
        // Causal mask, for every block when some block has a key after one of its rows
        // (a block whose rows all follow the run's last key is left unchanged by it).
        bool need_mask = false;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) need_mask = need_mask || first[cb] < tpos + 31;
        if (need_mask) {                                     // wave-uniform
#pragma unroll
            for (int cb = 0; cb < NC; ++cb)
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int key = (k < 4) ? 4 * c + k : 16 + 4 * c + (k - 4);
                    if (tpos + key > qpos[cb]) sv[cb][k] = -INFINITY;
                }
        }
        // this lane's maxima; a column's (over the four c-lanes) is needed only when some
        // score passes the running maximum by more than 2^8
        float mb[NC];
        bool grow[NC];
        bool any_grow = false;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            float x = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(sv[cb][0], sv[cb][1]), sv[cb][2]),
                                      __builtin_fmaxf(__builtin_fmaxf(sv[cb][3], sv[cb][4]), sv[cb][5]));
            mb[cb] = __builtin_fmaxf(x, __builtin_fmaxf(sv[cb][6], sv[cb][7]));
            grow[cb] = __any(mb[cb] * sl2 > m[cb] + 8.f);
            any_grow = any_grow || grow[cb];
        }
        if (any_grow) {                                      // wave-uniform, rare
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                if (!grow[cb]) continue;
                const float mbs = max_across_c(mb[cb]) * sl2;    // -inf stays -inf
                const float mn = __builtin_fmaxf(m[cb], mbs);
                const float mu = (mn == -INFINITY) ? 0.f : mn;
                const float alpha = fast_exp2(m[cb] - mu);   // 0 while nothing was seen
#pragma unroll
                for (int e = 0; e < DB; ++e) acc[cb][e] *= alpha;
                lacc[cb] *= alpha;
                m[cb] = mn;
            }
        }
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            const float mu = (m[cb] == -INFINITY) ? 0.f : m[cb];
            float pr[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) pr[k] = fast_exp2(fmaf(sv[cb][k], sl2, -mu));
            // bf16 weights: a rounded part plus its rounded remainder, both through the
            // matrix cores, so the value product sees about 16 significand bits of every
            // weight instead of bf16's 8 (with 8 bits a short row's output can miss the
            // decode bar by the weights' rounding alone).  fp16 weights keep 11 bits in
            // one part.
            if constexpr (kSplitWeights) {
                const uint2 w01 = split_pack2<S>(pr[0], pr[1]);
                const uint2 w23 = split_pack2<S>(pr[2], pr[3]);
                const uint2 w45 = split_pack2<S>(pr[4], pr[5]);
                const uint2 w67 = split_pack2<S>(pr[6], pr[7]);
                pop[cb] = make_uint4(w01.x, w23.x, w45.x, w67.x);
                pol[cb] = make_uint4(w01.y, w23.y, w45.y, w67.y);
            } else {
                pop[cb] = make_uint4(S::pack2(pr[0], pr[1]), S::pack2(pr[2], pr[3]),
                                     S::pack2(pr[4], pr[5]), S::pack2(pr[6], pr[7]));
            }
            // the column sums of the weights, on the matrix cores: an all-ones A operand
            // puts sum_k P[k][n] in every row of column n (the same parts the value
            // product uses)
            lacc[cb] = S::mfma_k32(ones, pop[cb], lacc[cb]);
        }
        // all rounded-part products first, then the remainders: the two products into one
        // accumulator are never back to back
#pragma unroll
        for (int e = 0; e < DB; ++e)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) acc[cb][e] = S::mfma_k32(vop[e], pop[cb], acc[cb][e]);
        if constexpr (kSplitWeights) {
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) lacc[cb] = S::mfma_k32(ones, pol[cb], lacc[cb]);
#pragma unroll
            for (int e = 0; e < DB; ++e)
#pragma unroll
                for (int cb = 0; cb < NC; ++cb) acc[cb][e] = S::mfma_k32(vop[e], pol[cb], acc[cb][e]);
        }
    };
    // one stage: its 32-key runs in turn, up to this wave's last position
    auto compute = [&](int j, int buf) {
#pragma unroll
        for (int h = 0; h < kPfRuns; ++h) {
            const int tpos = j * KT + 32 * h;
            if (h > 0 && tpos > wave_last) break;           // wave-uniform
            compute_half(tpos, lds_k[buf] + 32 * h * ROWB_K, lds_v[buf] + 32 * h * ROWB_V);
        }
    };

    // ---- this work-group's stages [j_lo, j_hi): all of them, or its split's equal run
    int nsplit = 1;                              // this row tile's splits
    if constexpr (!DENSE) {
        j_hi = nstages;
        if constexpr (SPLIT) {
            nsplit = tile_splits(pa.splits, nstages);
            if (split >= nsplit) return;         // the whole work-group: before any barrier
            const int per = (nstages + nsplit - 1) / nsplit;
            j_lo = min(nstages, split * per);
            j_hi = min(nstages, j_lo + per);
        }
    }
    // ---- pipeline: fetch stage j + 1 while computing stage j
    if (j_lo < j_hi) {
        if constexpr (!DENSE) {
            fetch_table(j_lo);
            fetch(j_lo);
        }
        stage_store(j_lo & 1);
        if (j_lo + 1 < j_hi) fetch_table(j_lo + 1);
    }
    for (int j = j_lo; j < j_hi; ++j) {
        if (j + 1 < j_hi) {
            fetch(j + 1);
            if (j + 2 < j_hi) fetch_table(j + 2);
        }
        __syncthreads();                         // stage j is in LDS buffer j & 1
        if (j < wave_stages) compute(j, j & 1);
        if (j + 1 < j_hi) stage_store((j + 1) & 1);      // its last readers passed the barrier
    }

    if constexpr (DENSE) {
        // partial results of the prefix, in half the bytes: each row's accumulator as 16-bit
        // integers q = round(acc * 2^(14 - x)), where 2^x bounds the row's largest magnitude
        // (|q| < 2^14, every element within 2^-15 of that bound), and (m, l, 2^(x - 14)).
        // Lane (n, c) holds elements 16 e + 4 c + rr of row n.
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            float mx = 0.f;
#pragma unroll
            for (int e = 0; e < DB; ++e)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) mx = fmaxf(mx, fabsf(acc[cb][e][rr]));
            mx = fmaxf(mx, __shfl_xor(mx, 16));      // the row's four lanes
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            int x = 0;
            (void)frexpf(mx, &x);                    // mx < 2^x (x = 0 for an all-zero row)
            const float to_q = ldexpf(1.f, 14 - x);
            const int r = row_base + cb * 16 + n;
            if (r >= rows) continue;
            const int t = tok[cb];
            const int g = r - t * G;
            const int64_t part = (static_cast<int64_t>(t) * a.num_q_heads + kvh * G + g) * pa.splits + split;
            int16_t* dst = reinterpret_cast<int16_t*>(pa.ws_acc) + part * D + 4 * c;
#pragma unroll
            for (int e = 0; e < DB; ++e) {
                const uint32_t lo = (static_cast<uint32_t>(__float2int_rn(acc[cb][e][0] * to_q)) & 0xffffu) |
                                    (static_cast<uint32_t>(__float2int_rn(acc[cb][e][1] * to_q)) << 16);
                const uint32_t hi = (static_cast<uint32_t>(__float2int_rn(acc[cb][e][2] * to_q)) & 0xffffu) |
                                    (static_cast<uint32_t>(__float2int_rn(acc[cb][e][3] * to_q)) << 16);
                *reinterpret_cast<uint2*>(dst + 16 * e) = make_uint2(lo, hi);
            }
            if (c == 0)
                *reinterpret_cast<float4*>(pa.ws_ml + 4 * part) =
                    make_float4(m[cb], lacc[cb][0], ldexpf(1.f, x - 14), 0.f);
        }
        return;
    } else if (SPLIT && nsplit > 1) {
        // partial results: lane (n, c) holds elements 16 e + 4 c + rr of row n; (m, l) as
        // the running maximum (base-2 units, -inf if no key was seen) and weight sum (a
        // tile with one split falls through to the output below)
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            const int r = row_base + cb * 16 + n;
            if (r >= rows) continue;
            const int t = tok[cb];
            if (q0 + t >= pa.num_tokens) continue;
            const int g = r - t * G;
            const int64_t part = (static_cast<int64_t>(q0 + t) * a.num_q_heads + kvh * G + g) * pa.splits + split;
            float* dst = pa.ws_acc + part * D + 4 * c;
#pragma unroll
            for (int e = 0; e < DB; ++e)
                *reinterpret_cast<float4*>(dst + 16 * e) =
                    make_float4(acc[cb][e][0], acc[cb][e][1], acc[cb][e][2], acc[cb][e][3]);
            if (c == 0) *reinterpret_cast<float2*>(pa.ws_ml + 2 * part) = make_float2(m[cb], lacc[cb][0]);
        }
        return;
    }

    // normalise and write: lane (n, c) holds elements 16 e + 4 c + rr of row n
#pragma unroll
    for (int cb = 0; cb < NC; ++cb) {
        const float lt = lacc[cb][0];
        const int r = row_base + cb * 16 + n;
        if (r >= rows) continue;
        const int t = tok[cb];
        const int g = r - t * G;
        const float inv = (qpos[cb] >= 0 && lt > 0.f) ? 1.f / lt : 0.f;
        uint16_t* dst = a.out + (static_cast<size_t>(q0 + t) * a.num_q_heads + kvh * G + g) * D + 4 * c;
#pragma unroll
        for (int e = 0; e < DB; ++e)
            *reinterpret_cast<uint2*>(dst + 16 * e) =
                make_uint2(S::pack2(acc[cb][e][0] * inv, acc[cb][e][1] * inv),
                           S::pack2(acc[cb][e][2] * inv, acc[cb][e][3] * inv));
    }
}

// Combines a split launch's partial results: O = sum_s w_s acc_s / sum_s w_s l_s with
// w_s = 2^(m_s - max m), summed in ascending s (deterministic).  The work-groups mirror
// the main kernel's row tiles (each tile's rows in groups of 16), so exactly the rows it
// computed are written; 16 lanes per row, D / 16 elements per lane, all of a row's
// partial results loaded at once.
template <class S, int D>
__global__ __launch_bounds__(256) void pa_prefill_merge(PrefillArgs pa) {
    constexpr int PER = D / 16;
    const DecodeArgs& a = pa.a;
    const int G = pa.group;
    const int subs = 2 * pa.waves;               // 16-row groups per row tile
    const int sub = static_cast<int>(blockIdx.x % subs);
    const int tile_id = static_cast<int>(blockIdx.x / subs);
    const int rt = pa.row_tiles - 1 - tile_id % pa.row_tiles;
    const int rest = tile_id / pa.row_tiles;
    const int kvh = rest % a.num_kv_heads;
    const int b = rest / a.num_kv_heads;
    const int q0 = pa.qstart[b];
    const int rows = (pa.qstart[b + 1] - q0) * G;
    const int tile_rows = 32 * pa.waves;
    // the tile's split count, as the main kernel takes it; a tile of one split wrote its
    // output itself
    const int nq = pa.qstart[b + 1] - q0;
    const int tile_last = clamped_length(a, b) - nq + (min(rows, (rt + 1) * tile_rows) - 1) / G;
    const int nsplit = tile_splits(pa.splits, tile_last >= 0 ? tile_last / (32 * kPfRuns) + 1 : 0);
    if (nsplit <= 1) return;
    const int r = rt * tile_rows + sub * 16 + static_cast<int>(threadIdx.x >> 4);
    if (r >= min(rows, (rt + 1) * tile_rows)) return;
    const int t = r / G;
    if (q0 + t >= pa.num_tokens) return;
    const int g = r - t * G;
    const int64_t row = static_cast<int64_t>(q0 + t) * a.num_q_heads + kvh * G + g;
    const int l16 = threadIdx.x & 15;
    const int S_ = nsplit;                       // of pa.splits slots per row
    const float2* ml = reinterpret_cast<const float2*>(pa.ws_ml) + row * pa.splits;
    const float* acc = pa.ws_acc + row * pa.splits * D + PER * l16;
    float2 v[kMaxPrefillSplits];
    float x[kMaxPrefillSplits][PER];
#pragma unroll
    for (int s = 0; s < kMaxPrefillSplits; ++s) {
        if (s < S_) {
            v[s] = ml[s];
#pragma unroll
            for (int e = 0; e < PER; e += 4) {
                const float4 q = *reinterpret_cast<const float4*>(acc + s * D + e);
                x[s][e] = q.x;
                x[s][e + 1] = q.y;
                x[s][e + 2] = q.z;
                x[s][e + 3] = q.w;
            }
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxPrefillSplits; ++s)
        if (s < S_) M = fmaxf(M, v[s].x);
    float A[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) A[e] = 0.f;
    float lsum = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxPrefillSplits; ++s) {
        if (s < S_) {
            const float w = (v[s].x == -INFINITY) ? 0.f : fast_exp2(v[s].x - M);
            lsum += w * v[s].y;
#pragma unroll
            for (int e = 0; e < PER; ++e) A[e] = fmaf(w, x[s][e], A[e]);
        }
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    uint32_t packed[PER / 2];
#pragma unroll
    for (int e = 0; e < PER; e += 2) packed[e / 2] = S::pack2(A[e] * inv, A[e + 1] * inv);
    uint16_t* dst = a.out + row * D + PER * l16;
    if constexpr (PER == 8) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    } else {
        *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
    }
}

template <class S, int D, bool KV8, bool SPLIT, bool DENSE = false>
void launch_main(const PrefillArgs& pa, unsigned grid, hipStream_t stream) {
    if (pa.waves == 8)
        hipLaunchKernelGGL((pa_prefill_mfma<S, D, 8, KV8, SPLIT, DENSE>), dim3(grid), dim3(64 * 8), 0, stream, pa);
    else
        hipLaunchKernelGGL((pa_prefill_mfma<S, D, 4, KV8, SPLIT, DENSE>), dim3(grid), dim3(64 * 4), 0, stream, pa);
}

template <class S, int D, bool KV8>
hipError_t launch_dense_t(const PrefillArgs& pa, hipStream_t stream) {
    const int64_t wgs = static_cast<int64_t>(pa.a.num_kv_heads) * pa.row_tiles * pa.splits;
    if (wgs <= 0) return hipSuccess;
    if (wgs > 0x7fffffff) return hipErrorInvalidValue;
    launch_main<S, D, KV8, true, true>(pa, static_cast<unsigned>(wgs), stream);
    return hipGetLastError();
}

template <class S, int D, bool KV8>
hipError_t launch_prefill_t(const PrefillArgs& pa, hipStream_t stream) {
    const int64_t wgs = static_cast<int64_t>(pa.a.batch) * pa.a.num_kv_heads * pa.row_tiles;
    if (wgs <= 0) return hipSuccess;
    if (wgs * std::max(pa.splits, 2 * pa.waves) > 0x7fffffff) return hipErrorInvalidValue;
    if (pa.splits > 1) {
        launch_main<S, D, KV8, true>(pa, static_cast<unsigned>(wgs * pa.splits), stream);
        hipLaunchKernelGGL((pa_prefill_merge<S, D>), dim3(static_cast<unsigned>(wgs * 2 * pa.waves)),
                           dim3(256), 0, stream, pa);
    } else {
        launch_main<S, D, KV8, false>(pa, static_cast<unsigned>(wgs), stream);
    }
    return hipGetLastError();
}

template <class S, int D, bool KV8>
int64_t resident_groups_t(int waves) {
    int dev = 0, cus = 0, blocks = 0;
    const void* k = waves == 8 ? reinterpret_cast<const void*>(&pa_prefill_mfma<S, D, 8, KV8, true>)
                               : reinterpret_cast<const void*>(&pa_prefill_mfma<S, D, 4, KV8, true>);
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, k, 64 * waves, 0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return static_cast<int64_t>(cus) * blocks;
}

}  // namespace

// 8 waves (256 rows, one work-group per CU) share each staged K/V tile between twice as
// many rows and halve each thread's staging work; 4 waves (128 rows, two work-groups per
// CU) keep twice as many work-groups for launches too small to fill the chip with 8.
// PAGEDKV_PREFILL_WAVES=4|8 forces the choice.
int prefill_waves_for(int64_t seq_heads, int64_t rows) {
    const char* e = getenv("PAGEDKV_PREFILL_WAVES");
    const int forced = e ? atoi(e) : 0;
    if (forced == 4 || forced == 8) return forced;
    const int64_t cus = device_cus() > 0 ? device_cus() : 256;
    return seq_heads * ((rows + 255) / 256) >= 2 * cus ? 8 : 4;
}

int64_t prefill_resident_groups(int kv_dtype, int io_dtype, int head_dim, int waves) {
    const bool kv8 = kv_dtype == KV_DTYPE_FP8_E4M3;
    if (io_dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return kv8 ? resident_groups_t<F16, 64, true>(waves) : resident_groups_t<F16, 64, false>(waves);
        if (head_dim == 128) return kv8 ? resident_groups_t<F16, 128, true>(waves) : resident_groups_t<F16, 128, false>(waves);
    } else if (io_dtype == KV_DTYPE_BF16) {
        if (head_dim == 64) return kv8 ? resident_groups_t<BF16, 64, true>(waves) : resident_groups_t<BF16, 64, false>(waves);
        if (head_dim == 128) return kv8 ? resident_groups_t<BF16, 128, true>(waves) : resident_groups_t<BF16, 128, false>(waves);
    }
    return 0;
}

hipError_t launch_prefill_dense(int kv_dtype, int io_dtype, int head_dim, const PrefillArgs& pa,
                                hipStream_t stream) {
    const bool kv8 = kv_dtype == KV_DTYPE_FP8_E4M3;
    if (io_dtype == KV_DTYPE_F16) {
        if (head_dim == 64) return kv8 ? launch_dense_t<F16, 64, true>(pa, stream) : launch_dense_t<F16, 64, false>(pa, stream);
        if (head_dim == 128) return kv8 ? launch_dense_t<F16, 128, true>(pa, stream) : launch_dense_t<F16, 128, false>(pa, stream);
    } else if (io_dtype == KV_DTYPE_BF16) {
        if (head_dim == 64) return kv8 ? launch_dense_t<BF16, 64, true>(pa, stream) : launch_dense_t<BF16, 64, false>(pa, stream);
        if (head_dim == 128) return kv8 ? launch_dense_t<BF16, 128, true>(pa, stream) : launch_dense_t<BF16, 128, false>(pa, stream);
    }
    return hipErrorInvalidValue;
}

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
