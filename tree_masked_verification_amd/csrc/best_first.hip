// best_first.hip -- best-first prefix trees from per-position draft marginals (gfx950).
//
// BASTION summary, sections 1-3: a block-diffusion drafter gives one marginal q_k per
// future position; a node at depth d (tokens x_1..x_d) scores rho = q_1(x_1)...q_d(x_d);
// best-first expansion adds, again and again, the highest-scoring node whose parent is in
// the tree; a controller keeps growing the tree while S(n) = A(n) L_AR / C(n) rises, with
// A(n) the sum of the first n scores.  Ties (our reading): the shallower node, then the
// smaller rank tuple, ranks per position by (q descending, token ascending); scores are
// fp64 products in depth order, so the result is exact and bit-identical to any correct
// implementation.
//
// Three launches:
//   1. every 32768-entry segment of every q row (512 threads, 64 entries each): its K
//      best entries, K = min(V, N_max).  Keys are (value bits << 32 | ~token), all
//      distinct.  The K-th largest of the threads' maxima is a threshold below which no
//      top-K entry lies, and at most K threads hold entries above it (at most 64 K
//      candidates).  Sorts keep one key per thread: partners within a wave trade keys
//      by lane shuffles, partners further apart through LDS.
//   2. every row: its segments' lists merged (sorted, one key per thread when they fit)
//      into the row's ranks.
//   3. every sequence, one wave: best-first over rank tuples.  A node's successors in the
//      order are its next sibling and its first child, so a frontier of at most N + 1
//      entries holds the next node at every step; it lives in registers, four slots per
//      lane, and each step is one wave-wide argmax.
#include "tmv_device.hpp"

namespace {

using tmv::kWave;

constexpr int kBfMaxN = 128;                        // nodes per tree
constexpr int kBfMaxD = 8;                          // positions (tree depth)
constexpr int kSegThreads = 512;
constexpr int kSegPer = 64;                         // entries per thread of a segment
constexpr int kSegLen = kSegThreads * kSegPer;      // entries per segment (32768)
constexpr int kMaxSegs = 8;                         // segments per row: V <= 262144
constexpr int kCand = kBfMaxN * kSegPer;            // candidates of a segment (at most)
constexpr int kRowKeys = kMaxSegs * kBfMaxN;        // keys a row merge sorts (at most)
constexpr int kBfBufferFlags = 0x00020000;          // raw buffer descriptor word 3 (gfx9 family)
constexpr uint32_t kNoEntry = 0xFFFFFFFFu;          // value bits of a missing entry (q <= 1 has bits <= 0x3F800000)
constexpr int kSlots = 4;                           // frontier slots per lane (4 * 64 >= kBfMaxN + 1)
constexpr int kRankBits = 7;                        // rank < 128
constexpr int kDepthShift = 56;                     // tuple key: depth << 56 | ranks, MSB first

// larger key = earlier rank (value descending, token ascending); 0 = no entry
__device__ __forceinline__ uint64_t rank_key(float v, int x) {
    return (static_cast<uint64_t>(__float_as_uint(v)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(x));
}

// sort keys[0, n) in descending order (n a power of two); every thread of the block calls it
__device__ void bitonic_desc(uint64_t *keys, int n) {
    for (int k = 2; k <= n; k <<= 1)
        for (int j = k >> 1; j > 0; j >>= 1) {
            __syncthreads();
            for (int i = threadIdx.x; i < n; i += blockDim.x) {
                const int l = i ^ j;
                if (l > i) {
                    const uint64_t a = keys[i], c = keys[l];
                    if ((i & k) == 0 ? a < c : a > c) {
                        keys[i] = c;
                        keys[l] = a;
                    }
                }
            }
        }
    __syncthreads();
}

// exclusive prefix sum over the block (kSegThreads threads); *total gets the sum
__device__ int block_exclusive_scan(int v, int *wave_sums, int *total) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    int incl = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += y;
    }
    __syncthreads();
    if (lane == kWave - 1) wave_sums[wv] = incl;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kSegThreads / kWave; ++w) {
        if (w < wv) before += wave_sums[w];
        all += wave_sums[w];
    }
    *total = all;
    return before + incl - v;
}

// Sort the block's keys, one per thread (kSegThreads of them), in descending order; returns
// the key that ends at position threadIdx.x.  Compare-exchange partners within a wave trade
// keys by lane shuffles; partners kWave or more apart trade through LDS (xbuf: two buffers
// of kSegThreads keys, alternated so each such stage needs one barrier).
__device__ uint64_t block_bitonic_desc(uint64_t key, uint64_t *xbuf) {
    const int i = threadIdx.x;
    int buf = 0;
    for (int k = 2; k <= kSegThreads; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            uint64_t other;
            if (j >= kWave) {
                uint64_t *x = xbuf + buf * kSegThreads;
                x[i] = key;
                __syncthreads();
                other = x[i ^ j];
                buf ^= 1;
            } else {
                const int lo = __shfl_xor(static_cast<int>(static_cast<uint32_t>(key)), j, kWave);
                const int hi = __shfl_xor(static_cast<int>(static_cast<uint32_t>(key >> 32)), j, kWave);
                other = (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
            }
            // of the pair (i, i ^ j), the lower position keeps the larger key when the
            // k-block runs descending ((i & k) == 0), the smaller one otherwise
            const bool take_max = ((i & j) == 0) == ((i & k) == 0);
            key = take_max ? (key > other ? key : other) : (key < other ? key : other);
        }
    }
    __syncthreads();
    return key;
}

__device__ __forceinline__ int pow2_at_least(int n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// ---- 1. the K best entries of each segment of each q row
__global__ void __launch_bounds__(kSegThreads)
bf_segment_kernel(int D, int V, int K, int nseg, const float *__restrict__ q, int64_t qsb, int64_t qsk,
                  uint64_t *__restrict__ seg_keys, int32_t *__restrict__ seg_bad)
{
    __shared__ uint64_t sh[kCand];
    __shared__ uint64_t xbuf[2 * kSegThreads];
    __shared__ uint64_t s_tau;
    __shared__ int wave_sums[kSegThreads / kWave];
    __shared__ int any_bad;
    const int tid = threadIdx.x;
    const int row = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int b = row / D, k = row % D;
    const float *qr = q + b * qsb + k * qsk;
    const int x0 = seg * kSegLen;
    if (tid == 0) any_bad = 0;

    // this thread's entries x0 + e * kSegThreads + tid (each load instruction is coalesced),
    // kept as value bits; an entry's key is rebuilt from its bits and position
    // (buffer loads: one vector offset, the entry's 4 KiB step in a scalar offset)
    const __amdgpu_buffer_rsrc_t qrs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(qr), 0, V * 4, kBfBufferFlags);
    uint32_t vb[kSegPer];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < kSegPer; ++e)
        vb[e] = __builtin_amdgcn_raw_buffer_load_b32(qrs, (x0 + tid) * 4, e * kSegThreads * 4, 0);
#pragma unroll
    for (int e = 0; e < kSegPer; ++e) {
        const int x = x0 + e * kSegThreads + tid;
        const float v = __uint_as_float(vb[e]);
        const bool ok = v >= 0.f && v <= 1.f;         // (false for NaN)
        bad = bad || (x < V && !ok);
        // -0.0 equals 0 and ranks as +0.0 (its raw bits would outrank every positive value)
        vb[e] = x < V && ok ? (vb[e] & 0x7fffffffu) : kNoEntry;
    }
    // the thread's largest key: largest value, then smallest token -- the first entry
    // holding the largest value bits (entries are in token order)
    uint32_t mv = kNoEntry;
    int me = 0;
#pragma unroll
    for (int e = 0; e < kSegPer; ++e) {
        const bool better = vb[e] != kNoEntry && (mv == kNoEntry || vb[e] > mv);
        mv = better ? vb[e] : mv;
        me = better ? e : me;
    }
    const uint64_t mx = mv == kNoEntry ? 0 : rank_key(__uint_as_float(mv), x0 + me * kSegThreads + tid);
    // does entry e's key reach (th, tl), the two halves of a key?  (32-bit compares only)
    auto reaches = [&](int e, uint32_t th, uint32_t tl) {
        const uint32_t lo = 0xFFFFFFFFu - static_cast<uint32_t>(x0 + e * kSegThreads + tid);
        return vb[e] != kNoEntry && (vb[e] > th || (vb[e] == th && lo >= tl));
    };
    // the K-th largest thread maximum: no top-K entry lies below it
    const uint64_t mx_sorted = block_bitonic_desc(mx, xbuf);
    if (tid == K - 1) s_tau = mx_sorted;
    if (bad) any_bad = 1;
    __syncthreads();
    const uint64_t tau = s_tau;
    // (tau = 0: fewer than K entries; every entry is a candidate)
    const uint32_t tau_hi = static_cast<uint32_t>(tau >> 32), tau_lo = static_cast<uint32_t>(tau);
    // candidates: entries >= tau (only the K threads whose maximum reaches tau hold any)
    int c = 0;
    uint32_t rm[kSegPer / 32] = {};              // bit e: entry e is a candidate
#pragma unroll
    for (int e = 0; e < kSegPer; ++e) rm[e >> 5] |= (reaches(e, tau_hi, tau_lo) ? 1u : 0u) << (e & 31);
#pragma unroll
    for (int w = 0; w < kSegPer / 32; ++w) c += __popc(rm[w]);
    int total = 0;
    const int off = block_exclusive_scan(c, wave_sums, &total);   // (its barriers also end the reads of sh)
    int o = off;
#pragma unroll
    for (int e = 0; e < kSegPer; ++e) {
        if (((rm[e >> 5] >> (e & 31)) & 1u) && o < kCand)
            sh[o++] = rank_key(__uint_as_float(vb[e]), x0 + e * kSegThreads + tid);
    }
    uint64_t *out = seg_keys + (static_cast<int64_t>(row) * nseg + seg) * K;
    if (total <= kSegThreads) {
        // (the usual case) one candidate per thread, the rest padded with 0
        __syncthreads();
        const uint64_t c = block_bitonic_desc(tid < total ? sh[tid] : 0, xbuf);
        if (tid < K) out[tid] = c;
    } else {
        const int n = pow2_at_least(total);
        for (int i = total + tid; i < n; i += kSegThreads) sh[i] = 0;
        bitonic_desc(sh, n);
        for (int r = tid; r < K; r += kSegThreads) out[r] = sh[r];
    }
    if (tid == 0) seg_bad[static_cast<int64_t>(row) * nseg + seg] = any_bad;
}

// ---- 2. each row's ranks from its segments' lists
__global__ void __launch_bounds__(kSegThreads)
bf_row_kernel(int K, int nseg, const uint64_t *__restrict__ seg_keys, const int32_t *__restrict__ seg_bad,
              int32_t *__restrict__ rank_tok, float *__restrict__ rank_val, int32_t *__restrict__ row_bad)
{
    __shared__ uint64_t xbuf[2 * kSegThreads];
    __shared__ uint64_t sh[kRowKeys];
    const int tid = threadIdx.x, row = blockIdx.x;
    const int m = nseg * K;                           // <= kRowKeys
    const uint64_t *keys = seg_keys + static_cast<int64_t>(row) * m;
    auto put = [&](int r, uint64_t key) {
        rank_tok[static_cast<int64_t>(row) * K + r] = static_cast<int32_t>(0xFFFFFFFFu - static_cast<uint32_t>(key));
        rank_val[static_cast<int64_t>(row) * K + r] = __uint_as_float(static_cast<uint32_t>(key >> 32));
    };
    if (m <= kSegThreads) {
        // one key per thread, the rest padded with 0
        const uint64_t c = block_bitonic_desc(tid < m ? keys[tid] : 0, xbuf);
        if (tid < K) put(tid, c);
    } else {
        const int n = pow2_at_least(m);
        for (int i = tid; i < n; i += kSegThreads) sh[i] = i < m ? keys[i] : 0;
        bitonic_desc(sh, n);
        for (int r = tid; r < K; r += kSegThreads) put(r, sh[r]);
    }
    if (tid == 0) {
        int bad = 0;
        for (int s = 0; s < nseg; ++s) bad |= seg_bad[static_cast<int64_t>(row) * nseg + s];
        row_bad[row] = bad;
    }
}

// ---- 3. best-first expansion and the budget controller, one wave per sequence
// does a come before b (score descending, then depth and rank tuple ascending)?
__device__ __forceinline__ bool before(double ra, uint64_t ka, double rb, uint64_t kb) {
    return ra > rb || (ra == rb && ka < kb);
}

// keep (r2, k2, s2) if it comes first (slot -1: no candidate; keys are distinct, so every
// lane makes the same choice)
__device__ __forceinline__ void take(double &r, uint64_t &k, int &s, double r2, uint64_t k2, int s2) {
    const bool t = s2 >= 0 && (s < 0 || before(r2, k2, r, k));
    r = t ? r2 : r;
    k = t ? k2 : k;
    s = t ? s2 : s;
}

__device__ __forceinline__ uint32_t lo32(uint64_t v) { return static_cast<uint32_t>(v); }
__device__ __forceinline__ uint32_t hi32(uint64_t v) { return static_cast<uint32_t>(v >> 32); }
__device__ __forceinline__ uint64_t join(uint32_t h, uint32_t l) { return (static_cast<uint64_t>(h) << 32) | l; }
__device__ __forceinline__ uint64_t dbits(double d) { return static_cast<uint64_t>(__double_as_longlong(d)); }
__device__ __forceinline__ double from_bits(uint64_t b) { return __longlong_as_double(static_cast<long long>(b)); }

// combine with the lane that DPP control CTRL reads from (within rows of 16 lanes)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ void dpp_take(double &r, uint64_t &k, int &s) {
    const uint64_t rb = dbits(r);
    const double r2 = from_bits(join(dpp32<CTRL>(hi32(rb)), dpp32<CTRL>(lo32(rb))));
    const uint64_t k2 = join(dpp32<CTRL>(hi32(k)), dpp32<CTRL>(lo32(k)));
    const int s2 = static_cast<int>(dpp32<CTRL>(static_cast<uint32_t>(s)));
    take(r, k, s, r2, k2, s2);
}

// combine the pairs of rows (16-lane swap) or of half-waves (32-lane swap): each swap hands
// every lane the values of both members of its pair
template <bool kHalves>
__device__ __forceinline__ void swap_take(double &r, uint64_t &k, int &s) {
    const uint64_t rb = dbits(r);
    uint32_t a0, a1, b0, b1, c0, c1, d0, d1, e0, e1;
    if constexpr (kHalves) {
        const auto a = __builtin_amdgcn_permlane32_swap(lo32(rb), lo32(rb), false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(hi32(rb), hi32(rb), false, false);
        const auto c = __builtin_amdgcn_permlane32_swap(lo32(k), lo32(k), false, false);
        const auto d = __builtin_amdgcn_permlane32_swap(hi32(k), hi32(k), false, false);
        const auto e = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(s), static_cast<uint32_t>(s), false, false);
        a0 = a[0]; a1 = a[1]; b0 = b[0]; b1 = b[1]; c0 = c[0]; c1 = c[1]; d0 = d[0]; d1 = d[1]; e0 = e[0]; e1 = e[1];
    } else {
        const auto a = __builtin_amdgcn_permlane16_swap(lo32(rb), lo32(rb), false, false);
        const auto b = __builtin_amdgcn_permlane16_swap(hi32(rb), hi32(rb), false, false);
        const auto c = __builtin_amdgcn_permlane16_swap(lo32(k), lo32(k), false, false);
        const auto d = __builtin_amdgcn_permlane16_swap(hi32(k), hi32(k), false, false);
        const auto e = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(s), static_cast<uint32_t>(s), false, false);
        a0 = a[0]; a1 = a[1]; b0 = b[0]; b1 = b[1]; c0 = c[0]; c1 = c[1]; d0 = d[0]; d1 = d[1]; e0 = e[0]; e1 = e[1];
    }
    r = from_bits(join(b0, a0));
    k = join(d0, c0);
    s = static_cast<int>(e0);
    take(r, k, s, from_bits(join(b1, a1)), join(d1, c1), static_cast<int>(e1));
}

// the earliest candidate of the wave, in every lane: xor 1 and xor 2 (quad permutes),
// quads (row half-mirror), half-rows (row mirror), rows, half-waves
__device__ __forceinline__ void wave_take(double &r, uint64_t &k, int &s) {
    dpp_take<0xB1>(r, k, s);        // quad_perm [1,0,3,2]
    dpp_take<0x4E>(r, k, s);        // quad_perm [2,3,0,1]
    dpp_take<0x141>(r, k, s);       // row_half_mirror
    dpp_take<0x140>(r, k, s);       // row_mirror
    swap_take<false>(r, k, s);
    swap_take<true>(r, k, s);
}

// the wave's largest value, in every lane (same exchange pattern as wave_take)
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, dpp32<0xB1>(v));
    v = mx(v, dpp32<0x4E>(v));
    v = mx(v, dpp32<0x141>(v));
    v = mx(v, dpp32<0x140>(v));
    const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = mx(a[0], a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return mx(c[0], c[1]);
}

__global__ void __launch_bounds__(kWave)
bf_expand_kernel(int D, int K, int N_max, const int32_t *__restrict__ rank_tok, const float *__restrict__ rank_val,
                 const int32_t *__restrict__ row_bad, const double *__restrict__ cost, double l_ar,
                 int32_t *__restrict__ parents, int32_t *__restrict__ tokens, int32_t *__restrict__ n_nodes,
                 double *__restrict__ rho, int32_t *__restrict__ status)
{
    __shared__ float rv[kBfMaxD][kBfMaxN];
    __shared__ int32_t rt[kBfMaxD][kBfMaxN];
    __shared__ int32_t out_par[kBfMaxN + 1], out_tok[kBfMaxN + 1];
    __shared__ double out_rho[kBfMaxN + 1];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int R = N_max + 1;
    int32_t *pb = parents + static_cast<int64_t>(b) * R;
    int32_t *tb = tokens + static_cast<int64_t>(b) * R;
    double *rb = rho + static_cast<int64_t>(b) * R;

    const int st = status[b];
    int bad = 0;
    for (int k = 0; k < D; ++k) bad |= row_bad[static_cast<int64_t>(b) * D + k];
    if (st != TMV_OK || bad) {
        for (int j = lane; j < R; j += kWave) {
            pb[j] = 0;
            tb[j] = 0;
            rb[j] = j == 0 ? 1.0 : 0.0;
        }
        if (lane == 0) {
            n_nodes[b] = 0;
            if (st == TMV_OK) status[b] = TMV_ERR_INPUT;
        }
        return;
    }
    for (int i = lane; i < D * K; i += kWave) {
        rv[i / K][i % K] = rank_val[static_cast<int64_t>(b) * D * K + i];
        rt[i / K][i % K] = rank_tok[static_cast<int64_t>(b) * D * K + i];
    }
    __syncthreads();

    // frontier slot s lives in lane s % 64, register s / 64 (one array per field); slot 0
    // starts as the best child of the root
    double f_rho[kSlots], f_prho[kSlots];
    uint64_t f_key[kSlots];
    int f_par[kSlots];
    bool f_live[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
        const bool first = lane == 0 && j == 0;
        f_rho[j] = first ? static_cast<double>(rv[0][0]) : 0.0;
        f_prho[j] = 1.0;
        f_key[j] = 1ull << kDepthShift;
        f_par[j] = 0;
        f_live[j] = first;
    }
    int used = 1;                                    // slots handed out so far (wave-uniform)
    int n = 0;
    while (n < N_max) {
        // the earliest live slot.  Scores are positive doubles, so their upper 32 bits order
        // them up to ties there: the wave's largest upper word (+1, 0 for a dead slot) picks
        // the slot when one slot alone holds it; otherwise the exact comparison runs over
        // the slots that hold it.
        uint32_t top = 0;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            const uint32_t h = f_live[j] ? hi32(dbits(f_rho[j])) + 1 : 0;
            top = h > top ? h : top;
        }
        top = __builtin_amdgcn_readfirstlane(wave_max_u32(top));
        if (top == 0) break;                         // every possible node is in the tree
        uint64_t hold[kSlots];
        int n_hold = 0, js = 0;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            hold[j] = __ballot(f_live[j] && hi32(dbits(f_rho[j])) + 1 == top);
            n_hold += __popcll(hold[j]);
            js = hold[j] != 0 ? j : js;
        }
        int owner;
        if (n_hold == 1) {
            owner = __ffsll(static_cast<long long>(hold[js])) - 1;
        } else {
            double br = 0.0;
            uint64_t bk = 0;
            int bs = -1;
#pragma unroll
            for (int j = 0; j < kSlots; ++j)
                if ((hold[j] >> lane) & 1ull) take(br, bk, bs, f_rho[j], f_key[j], j * kWave + lane);
            wave_take(br, bk, bs);
            bs = __builtin_amdgcn_readfirstlane(bs);
            owner = bs % kWave;
            js = bs / kWave;
        }
        double prho = 0.0, br = 0.0;
        uint64_t bk = 0;
        int par = 0;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            prho = j == js ? f_prho[j] : prho;
            br = j == js ? f_rho[j] : br;
            bk = j == js ? f_key[j] : bk;
            par = j == js ? f_par[j] : par;
        }
        prho = from_bits(join(__builtin_amdgcn_readlane(hi32(dbits(prho)), owner),
                              __builtin_amdgcn_readlane(lo32(dbits(prho)), owner)));
        br = from_bits(join(__builtin_amdgcn_readlane(hi32(dbits(br)), owner),
                            __builtin_amdgcn_readlane(lo32(dbits(br)), owner)));
        bk = join(__builtin_amdgcn_readlane(hi32(bk), owner), __builtin_amdgcn_readlane(lo32(bk), owner));
        par = __builtin_amdgcn_readlane(par, owner);
        ++n;
        const int d = static_cast<int>(bk >> kDepthShift);
        const int sh_r = kDepthShift - kRankBits * d;    // bit offset of the last position's rank
        const int r = static_cast<int>((bk >> sh_r) & ((1u << kRankBits) - 1));
        if (lane == 0) {
            out_par[n] = par;
            out_tok[n] = rt[d - 1][r];
            out_rho[n] = br;
        }
        // successors: the next sibling (same parent, next rank) and the first child
        const bool has_sib = r + 1 < K, has_child = d < D;
        const double sib_rho = prho * static_cast<double>(rv[d - 1][has_sib ? r + 1 : r]);
        const uint64_t sib_key = bk + (1ull << sh_r);
        const double child_rho = br * static_cast<double>(rv[has_child ? d : 0][0]);
        const uint64_t child_key = (static_cast<uint64_t>(d + 1) << kDepthShift) | (bk & ((1ull << kDepthShift) - 1));
        // the popped slot takes the sibling (else the child, else it dies); a child next to
        // a sibling takes a new slot
        const int new_slot = used;
        const bool use_new = has_sib && has_child;
        if (use_new) ++used;
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            const bool here = lane == owner && j == js;
            const bool fresh = use_new && lane == new_slot % kWave && j == new_slot / kWave;
            const bool to_sib = here && has_sib;
            const bool to_child = fresh || (here && !has_sib && has_child);
            f_rho[j] = to_sib ? sib_rho : to_child ? child_rho : f_rho[j];
            f_prho[j] = to_sib ? prho : to_child ? br : f_prho[j];
            f_key[j] = to_sib ? sib_key : to_child ? child_key : f_key[j];
            f_par[j] = to_sib ? par : to_child ? n : f_par[j];
            f_live[j] = (to_sib || to_child) ? true : (here ? false : f_live[j]);
        }
    }
    __syncthreads();

    // the controller: the first n whose successor lowers S(n) = A(n) L_AR / C(n)
    int keep = n;
    if (cost != nullptr && lane == 0) {
        double a = 0.0, s_prev = 0.0;
        for (int m = 1; m <= n; ++m) {
            a += out_rho[m];
            const double s = a * l_ar / cost[m - 1];
            if (m > 1 && s < s_prev) {
                keep = m - 1;
                break;
            }
            s_prev = s;
        }
    }
    keep = __shfl(keep, 0, kWave);
    for (int j = lane; j < R; j += kWave) {
        const bool in = j >= 1 && j <= keep;
        pb[j] = in ? out_par[j] : 0;
        tb[j] = in ? out_tok[j] : 0;
        rb[j] = j == 0 ? 1.0 : in ? out_rho[j] : 0.0;
    }
    if (lane == 0) n_nodes[b] = keep;
}

// workspace: seg_keys [rows][nseg][K] u64 | seg_bad [rows][nseg] | rank_tok [rows][K] |
// rank_val [rows][K] f32 | row_bad [rows]
struct BfLayout {
    size_t seg_keys, seg_bad, rank_tok, rank_val, row_bad, total;
};

size_t bf_align(size_t x) { return (x + 255) / 256 * 256; }

BfLayout bf_layout(int B, int D, int V, int N_max) {
    const size_t rows = static_cast<size_t>(B) * D;
    const size_t K = static_cast<size_t>(V < N_max ? V : N_max);
    const size_t nseg = (static_cast<size_t>(V) + kSegLen - 1) / kSegLen;
    BfLayout l;
    l.seg_keys = 0;
    l.seg_bad = l.seg_keys + bf_align(rows * nseg * K * sizeof(uint64_t));
    l.rank_tok = l.seg_bad + bf_align(rows * nseg * sizeof(int32_t));
    l.rank_val = l.rank_tok + bf_align(rows * K * sizeof(int32_t));
    l.row_bad = l.rank_val + bf_align(rows * K * sizeof(float));
    l.total = l.row_bad + bf_align(rows * sizeof(int32_t));
    return l;
}

}  // namespace

extern "C" size_t tmv_tree_best_first_workspace(int B, int D, int V, int N_max)
{
    if (B <= 0 || D <= 0 || V <= 0 || N_max <= 0) return 256;
    return bf_layout(B, D, V, N_max).total;
}

extern "C" int tmv_tree_best_first(int B, int D, int V, int N_max, const float *q, int64_t q_stride_b,
                                   int64_t q_stride_k, const double *cost, double l_ar, int32_t *parents,
                                   int32_t *tokens, int32_t *n_nodes, double *rho, int32_t *status,
                                   void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 0 || D < 1 || D > kBfMaxD || V < 1 || V > kMaxSegs * kSegLen || N_max < 1 || N_max > kBfMaxN)
        return TMV_ERR_ARG;
    if (q_stride_b < 0 || q_stride_k < 0) return TMV_ERR_ARG;
    if (B == 0) return TMV_OK;
    if (!q || !parents || !tokens || !n_nodes || !rho || !status || !workspace) return TMV_ERR_ARG;
    const BfLayout l = bf_layout(B, D, V, N_max);
    if (workspace_bytes < l.total || (reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return TMV_ERR_ARG;
    const int K = V < N_max ? V : N_max;
    const int nseg = (V + kSegLen - 1) / kSegLen;
    const int64_t rows = static_cast<int64_t>(B) * D;
    if (rows * nseg > 0x7fffffff) return TMV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    uint64_t *seg_keys = reinterpret_cast<uint64_t *>(ws + l.seg_keys);
    int32_t *seg_bad = reinterpret_cast<int32_t *>(ws + l.seg_bad);
    int32_t *rank_tok = reinterpret_cast<int32_t *>(ws + l.rank_tok);
    float *rank_val = reinterpret_cast<float *>(ws + l.rank_val);
    int32_t *row_bad = reinterpret_cast<int32_t *>(ws + l.row_bad);
    hipLaunchKernelGGL(bf_segment_kernel, dim3(static_cast<unsigned>(rows * nseg)), dim3(kSegThreads), 0, s, D, V, K,
                       nseg, q, q_stride_b, q_stride_k, seg_keys, seg_bad);
    hipLaunchKernelGGL(bf_row_kernel, dim3(static_cast<unsigned>(rows)), dim3(kSegThreads), 0, s, K, nseg, seg_keys,
                       seg_bad, rank_tok, rank_val, row_bad);
    hipLaunchKernelGGL(bf_expand_kernel, dim3(B), dim3(kWave), 0, s, D, K, N_max, rank_tok, rank_val, row_bad, cost,
                       l_ar, parents, tokens, n_nodes, rho, status);
    return tmv_host::launch_status(hipGetLastError());
}
