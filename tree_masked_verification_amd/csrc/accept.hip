// accept.hip -- choosing the accepted path of a verified draft tree (gfx950).
//
// GREEDY: the teacher's argmax of every live row, then the deepest node whose whole
//   path matches those choices (Medusa section of "Speculative Decoding Hierarquico":
//   the longest valid branch is kept).  The row scans are the HBM-bound part: one
//   workgroup per (sequence, row, vocabulary chunk) reads its chunk with 16-byte loads
//   and reduces a 64-bit key (order-preserving value bits << 32 | ~index), so max() gives
//   the largest value and, on ties, the smallest index.  A second kernel (one
//   workgroup per sequence, ordered after the scan on the stream) merges the chunk keys
//   and picks the path -- no cross-workgroup synchronisation inside a kernel.
// SAMPLE: modified rejection sampling (same page, its rejection-sampling section and
//   FAQ), children of the current node tried in ascending id against the running
//   residual.  Exact integer fixed point, so the result is bit-identical to any correct
//   implementation: one workgroup walks one sequence; every full-row pass (row sums,
//   residual update, inverse-CDF draw) is a block-wide integer reduction or scan.
#include "tmv_device.hpp"

namespace {

using tmv::kWave;
using tmv::u128;

// ============================================================== greedy
constexpr int kScanThreads = 256;
constexpr int kScanChunk = 4096;          // vocabulary entries per workgroup (four 16-byte loads per thread)
constexpr uint64_t kNanKey = ~0ull;       // a chunk with a NaN reports the all-ones key

__device__ __forceinline__ uint32_t order_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void scan_one(float v, int idx, uint64_t &best, bool &nan) {
    if (v != v) nan = true;
    const uint64_t key = (static_cast<uint64_t>(order_bits(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(idx));
    best = key > best ? key : best;
}

template <int DT>
__global__ void __launch_bounds__(kScanThreads)
greedy_scan_kernel(int M_max, int V, int nchunk, const void *__restrict__ teacher, int64_t sb, int64_t sr,
                   const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ depth,
                   const int32_t *__restrict__ status, uint64_t *__restrict__ keys)
{
    __shared__ uint64_t red[kScanThreads / kWave];
    const int R = M_max + 1;
    const int chunk = blockIdx.x % nchunk;
    const int u = (blockIdx.x / nchunk) % R;
    const int b = blockIdx.x / (nchunk * R);
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    // The row's loads go out before the words that decide whether the row is live have
    // returned: every (b, u, chunk) of the grid addresses the teacher tensor in bounds, so
    // a dead row only costs bandwidth, and a live one saves a round trip.
    const int M = n_nodes[b];
    const int st = status[b];
    const int dp = u > 0 ? depth[static_cast<int64_t>(b) * R + u] : 1;

    const int x0 = chunk * kScanChunk;
    const int x1 = min(V, x0 + kScanChunk);
    uint64_t best = 0;
    bool nan = false;
    if constexpr (DT == TMV_F32) {
        const float *row = static_cast<const float *>(teacher) + b * sb + static_cast<int64_t>(u) * sr;
        constexpr int kPer = kScanChunk / (4 * kScanThreads);        // float4 per thread
        if (x1 - x0 == kScanChunk && ((reinterpret_cast<uintptr_t>(row + x0) & 15u) == 0)) {
            const float4 *r4 = reinterpret_cast<const float4 *>(row + x0);
            float4 f[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) f[i] = r4[tid + i * kScanThreads];
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int x = x0 + 4 * (tid + i * kScanThreads);
                scan_one(f[i].x, x, best, nan);
                scan_one(f[i].y, x + 1, best, nan);
                scan_one(f[i].z, x + 2, best, nan);
                scan_one(f[i].w, x + 3, best, nan);
            }
        } else {
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
            for (int x = x0 + tid; x < x1; x += kScanThreads) scan_one(row[x], x, best, nan);
        }
    } else {
        const uint16_t *row = static_cast<const uint16_t *>(teacher) + b * sb + static_cast<int64_t>(u) * sr;
        constexpr int kPer = kScanChunk / (8 * kScanThreads);        // 8 bf16 per thread and load
        if (x1 - x0 == kScanChunk && ((reinterpret_cast<uintptr_t>(row + x0) & 15u) == 0)) {
            const uint4 *r8 = reinterpret_cast<const uint4 *>(row + x0);
            uint4 h[kPer];
#pragma unroll
            for (int i = 0; i < kPer; ++i) h[i] = r8[tid + i * kScanThreads];
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int x = x0 + 8 * (tid + i * kScanThreads);
                const uint32_t w[4] = {h[i].x, h[i].y, h[i].z, h[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    scan_one(__uint_as_float(w[e] << 16), x + 2 * e, best, nan);
                    scan_one(__uint_as_float(w[e] & 0xffff0000u), x + 2 * e + 1, best, nan);
                }
            }
        } else {
            if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
            for (int x = x0 + tid; x < x1; x += kScanThreads) scan_one(tmv::bf16_to_f32(row[x]), x, best, nan);
        }
    }
    if (nan) best = kNanKey;
    best = tmv::wave_max_u64(best);
    if (lane == 0) red[wv] = best;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = red[0];
        for (int w = 1; w < kScanThreads / kWave; ++w) k = red[w] > k ? red[w] : k;
        keys[(static_cast<int64_t>(b) * R + u) * nchunk + chunk] = k;
    }
}

// One workgroup per sequence, after the scan: merge the chunk keys of every live row into
// t(u), check the draft tokens, mark matching nodes and pick the deepest (smallest id).
__global__ void __launch_bounds__(kScanThreads)
greedy_select_kernel(int M_max, int D_max, int V, int nchunk, const int32_t *__restrict__ tokens,
                     const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ anc,
                     const int32_t *__restrict__ depth, int32_t *__restrict__ status,
                     int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                     int32_t *__restrict__ next_token, const uint64_t *__restrict__ keys)
{
    constexpr int kKeyBatch = 32;                  // chunk keys per row fetched at once
    constexpr int kAncBatch = 8;                   // ancestor entries per node fetched at once
    __shared__ int32_t tsel[129], tok_sh[129];
    __shared__ int bad;
    __shared__ uint64_t best_node[kScanThreads / kWave];
    const int R = M_max + 1, W = D_max + 1;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;

    // one round trip: sequence scalars, this thread's row of keys, token, depth and
    // first ancestor entries (indices clamped into the tables)
    const int M = n_nodes[b];
    const int st_in = status[b];
    const int row = tid < R ? tid : R - 1;
    const int64_t rb = static_cast<int64_t>(b) * R + row;
    uint64_t kb[kKeyBatch];
#pragma unroll
    for (int c = 0; c < kKeyBatch; ++c) kb[c] = c < nchunk ? keys[rb * nchunk + c] : 0;
    const int tok = tokens[rb];
    const int dep = row > 0 ? depth[rb] : 0;
    int a8[kAncBatch];
    const int32_t *arow = anc + rb * W;
#pragma unroll
    for (int k = 0; k < kAncBatch; ++k) a8[k] = arow[k < W ? k : W - 1];

    // a node count outside [0, M_max] cannot come with an OK status from the build stage;
    // it is rejected here so that no row beyond the tables is ever addressed
    const int st = (st_in == TMV_OK && (M < 0 || M > M_max)) ? TMV_ERR_INPUT : st_in;
    int32_t *pth = path + static_cast<int64_t>(b) * D_max;
    if (tid == 0) bad = st != TMV_OK;
    if (tid < R) tok_sh[tid] = tok;
    __syncthreads();
    const bool row_live = st == TMV_OK && tid < R && tid <= M && (tid == 0 || dep >= 1);
    if (row_live) {
        uint64_t k = 0;
#pragma unroll
        for (int c = 0; c < kKeyBatch; ++c) k = kb[c] > k ? kb[c] : k;
        for (int c = kKeyBatch; c < nchunk; ++c) {
            const uint64_t kc = keys[rb * nchunk + c];
            k = kc > k ? kc : k;
        }
        if (k == kNanKey) bad = 1;
        tsel[tid] = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(k & 0xffffffffu));
        if (tid > 0 && (tok < 0 || tok >= V)) bad = 1;
    }
    __syncthreads();
    if (bad) {
        for (int j = tid; j < D_max; j += kScanThreads) pth[j] = 0;
        if (tid == 0) {
            accept_len[b] = 0;
            next_token[b] = 0;
            if (st_in == TMV_OK) status[b] = TMV_ERR_INPUT;
        }
        return;
    }
    // node i matches iff every node c on its path has token == t(parent(c)); the chosen
    // node maximises (depth, -id): key = depth << 8 | (255 - id)
    uint64_t key = 0;
    if (tid >= 1 && tid <= M && dep >= 1) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < kAncBatch; ++k) {
            if (k < dep) {
                const int parent = k + 1 < kAncBatch ? a8[k + 1] : arow[k + 1];
                ok = ok && tok_sh[a8[k]] == tsel[k + 1 < dep ? parent : 0];
            }
        }
        for (int k = kAncBatch; k < dep && ok; ++k)
            ok = tok_sh[arow[k]] == tsel[arow[k + 1]];
        if (ok) key = (static_cast<uint64_t>(dep) << 8) | static_cast<uint64_t>(255 - tid);
    }
    key = tmv::wave_max_u64(key);
    if (lane == 0) best_node[wv] = key;
    __syncthreads();
    if (tid == 0) {
        uint64_t k = best_node[0];
        for (int w = 1; w < kScanThreads / kWave; ++w) k = best_node[w] > k ? best_node[w] : k;
        const int star = k ? 255 - static_cast<int>(k & 255u) : 0;
        const int dstar = static_cast<int>(k >> 8);
        best_node[0] = (static_cast<uint64_t>(dstar) << 32) | static_cast<uint32_t>(star);
        accept_len[b] = dstar;
        next_token[b] = tsel[star];
    }
    __syncthreads();
    const int dstar = static_cast<int>(best_node[0] >> 32), star = static_cast<int>(best_node[0] & 0xffffffffu);
    for (int j = tid; j < D_max; j += kScanThreads)
        pth[j] = j < dstar ? anc[(static_cast<int64_t>(b) * R + star) * W + (dstar - 1 - j)] : 0;
}

// ============================================================== sampling
// K workgroups walk each sequence together, each owning a contiguous slice of the
// vocabulary: every full-row pass is split over the K slices, and the slices' exact
// partial sums meet at a per-sequence barrier (device-scope atomics in the workspace,
// bounded wait).  All K take the same decisions from the same sums and random words; the
// stored residual of a slice is only ever read and written by its owner, and the owner
// of the next child's token publishes that token's weight with its partial sum.
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kMaxSlices = 16;                 // workgroups per sequence
constexpr uint64_t kSyncSpinTicks = 200000;    // 2 ms at the 100 MHz s_memrealtime clock
constexpr int kFlagBad = 1;                    // an entry outside [0, 1] in a scanned row
constexpr int kFlagTimeout = 2;                // a workgroup stopped waiting for the others

// block-wide exact sum of one u128 per thread (result broadcast to every thread)
__device__ u128 block_sum_u128(u128 v, u128 *sh) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    v = tmv::wave_sum_u128(v);
    __syncthreads();
    if (lane == 0) sh[wv] = v;
    __syncthreads();
    u128 t = 0;
    for (int w = 0; w < kSampleWaves; ++w) t += sh[w];
    return t;
}

__device__ int block_or(int v, int *sh) {
    __syncthreads();
    if (threadIdx.x == 0) *sh = 0;
    __syncthreads();
    if (v) atomicOr(sh, 1);
    __syncthreads();
    return *sh;
}

// floor(p * 2^32) for p in [0,1]; flags entries outside [0,1] (and NaN)
__device__ __forceinline__ uint64_t quantise(float p, int &bad) {
    // floor(p * 2^32) from the fp32 bits: p = m * 2^(e - 150) with m the 24-bit significand,
    // so p * 2^32 = m * 2^(e - 118), exact in integers (the same value as in fp64)
    const uint32_t u = __float_as_uint(p);
    if (u > 0x3F800000u) {                     // above 1, negative, infinite or NaN
        if (u != 0x80000000u) bad = 1;         // (-0 is zero)
        return 0;
    }
    const uint32_t e = u >> 23;
    const uint64_t m = (u & 0x7FFFFFu) | 0x800000u;
    if (e >= 118) return m << (e - 118);       // e <= 127: at most 2^32
    const uint32_t sh = 118 - e;
    return sh >= 24 ? 0 : m >> sh;             // zero and subnormals give 0
}

// Per-sequence synchronisation block of the workspace; arrival and leave counts are zero
// between calls (the last workgroup to leave returns them to zero).
struct SeqSync {
    uint64_t arrive;                         // barrier arrivals in this call
    uint64_t leave;                          // workgroups done with this call
    uint64_t pad[14];
    uint64_t rec[2][kMaxSlices][4];          // by phase parity and slice: sum lo, sum hi, extra, flags
};

struct SeqView {
    u128 own;        // this slice's sum
    u128 total;      // sum over the slices
    u128 before;     // sum over the slices before this one
    uint64_t extra;  // the value published by the chosen owner slice
    int flags;       // OR of the slices' flags, plus kFlagTimeout if this workgroup gave up
};

struct SyncLds {
    u128 red[kSampleWaves];
    int flag;
    int res_flags;
    uint64_t res[5];
};

// Sum `local` over the block and then over the K slices of the sequence.  Every thread
// of the block calls it; `phase` counts the calls and must advance alike in all K.
__device__ SeqView seq_reduce(SeqSync *ss, int K, int k, int &phase, u128 local, uint64_t extra, int owner,
                              int flags, SyncLds &L)
{
    const u128 wg = block_sum_u128(local, L.red);
    const int fl = block_or(flags, &L.flag);
    const int slot = phase & 1;
    ++phase;
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        int timed_out = 0;
        if (lane == 0) {
            uint64_t *r = ss->rec[slot][k];
            __hip_atomic_store(r + 0, static_cast<uint64_t>(wg), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(r + 1, static_cast<uint64_t>(wg >> 64), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(r + 2, extra, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(r + 3, static_cast<uint64_t>(fl), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __builtin_amdgcn_s_waitcnt(0);                 // the record is out before the count
            __hip_atomic_fetch_add(&ss->arrive, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t target = static_cast<uint64_t>(K) * phase;
            const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
            while (__hip_atomic_load(&ss->arrive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                if (__builtin_amdgcn_s_memrealtime() - t0 > kSyncSpinTicks) { timed_out = 1; break; }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);          // the record reads stay after the wait
        u128 v = 0;
        uint64_t ex = 0;
        int f = 0;
        if (lane < K) {
            const uint64_t *rj = ss->rec[slot][lane];
            const uint64_t lo = __hip_atomic_load(rj + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t hi = __hip_atomic_load(rj + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ex = __hip_atomic_load(rj + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            f = static_cast<int>(__hip_atomic_load(rj + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            v = (static_cast<u128>(hi) << 64) | lo;
        }
        const u128 tot = tmv::wave_sum_u128(v);
        const u128 bef = tmv::wave_sum_u128(lane < k ? v : 0);
        const uint32_t ex_lo = __shfl(static_cast<uint32_t>(ex), owner, kWave);
        const uint32_t ex_hi = __shfl(static_cast<uint32_t>(ex >> 32), owner, kWave);
        for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o, kWave);
        if (lane == 0) {
            L.res[0] = static_cast<uint64_t>(tot);
            L.res[1] = static_cast<uint64_t>(tot >> 64);
            L.res[2] = static_cast<uint64_t>(bef);
            L.res[3] = static_cast<uint64_t>(bef >> 64);
            L.res[4] = (static_cast<uint64_t>(ex_hi) << 32) | ex_lo;
            L.res_flags = f | (timed_out ? kFlagTimeout : 0);
        }
    }
    __syncthreads();
    SeqView r;
    r.own = wg;
    r.total = (static_cast<u128>(L.res[1]) << 64) | L.res[0];
    r.before = (static_cast<u128>(L.res[3]) << 64) | L.res[2];
    r.extra = L.res[4];
    r.flags = L.res_flags;
    return r;
}

// the workgroup is done with the call; the last of the K returns the counts to zero
__device__ void seq_leave(SeqSync *ss, int K) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __builtin_amdgcn_s_waitcnt(0);
        const uint64_t l = __hip_atomic_fetch_add(&ss->leave, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (l == static_cast<uint64_t>(K) - 1) {
            __hip_atomic_store(&ss->arrive, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ss->leave, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

struct Dist {       // the working distribution W of the walk
    const float *row;    // W(x) = floor(row[x] * 2^32) >> shift when stored == false
    int shift;
    bool stored;         // W lives in the workspace array
    uint64_t S;          // sum of W, renormalised to at most 48 bits
};

// A pass over the slice [x_lo, x_hi) strided over the block: x is visited by thread
// (x - x_lo) mod kSampleThreads, and each thread has kPassBatch loads in flight --
// load(x) for a whole batch goes out before body(x, value) runs on any of them.  (x and
// its value stay in one thread, so a body may overwrite what its own load read.)
constexpr int kPassBatch = 8;
template <class Load, class Body>
__device__ __forceinline__ void strided_pass(int x_lo, int x_hi, Load load, Body body) {
    for (int x0 = x_lo + static_cast<int>(threadIdx.x); x0 < x_hi; x0 += kPassBatch * kSampleThreads) {
        decltype(load(0)) v[kPassBatch];
#pragma unroll
        for (int j = 0; j < kPassBatch; ++j) {
            const int x = x0 + j * kSampleThreads;
            if (x < x_hi) v[j] = load(x);
        }
#pragma unroll
        for (int j = 0; j < kPassBatch; ++j) {
            const int x = x0 + j * kSampleThreads;
            if (x < x_hi) body(x, v[j]);
        }
    }
}

// the working distribution's raw entry at x (a stored W, or the bits of the p value)
// together with the draft's q(x)
struct RowPair {
    uint64_t a;
    float q;
};

__global__ void __launch_bounds__(kSampleThreads)
sample_walk_kernel(int M_max, int D_max, int V, int K,
                   const int32_t *__restrict__ tokens,
                   const float *__restrict__ p, int64_t psb, int64_t psr,
                   const float *__restrict__ q, int64_t qsb, int64_t qsr,
                   uint64_t seed, uint64_t step,
                   const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ anc,
                   const int32_t *__restrict__ depth, int32_t *__restrict__ status,
                   int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                   int32_t *__restrict__ next_token, uint64_t *__restrict__ wsW, SeqSync *__restrict__ sync)
{
    __shared__ SyncLds L;
    __shared__ int kids[129];
    __shared__ int nkids;
    __shared__ int kid_count[kSampleWaves];
    __shared__ u128 scan_sh[kSampleWaves];
    __shared__ int draw_tok;

    const int b = blockIdx.x / K, k = blockIdx.x % K, tid = threadIdx.x;
    const int x_lo = static_cast<int>(static_cast<int64_t>(V) * k / K);
    const int x_hi = static_cast<int>(static_cast<int64_t>(V) * (k + 1) / K);
    auto owner_of = [&](int x) {                 // the slice holding token x
        int o = static_cast<int>(static_cast<int64_t>(x) * K / V);
        while (o + 1 < K && static_cast<int64_t>(V) * (o + 1) / K <= x) ++o;
        while (o > 0 && static_cast<int64_t>(V) * o / K > x) --o;
        return o;
    };
    SeqSync *ss = sync + b;
    int phase = 0;
    const int R = M_max + 1, W = D_max + 1;
    const int M = n_nodes[b];
    int32_t *pth = path + static_cast<int64_t>(b) * D_max;
    uint64_t *w = wsW + static_cast<int64_t>(b) * V;
    const int st_in = status[b];
    const int st = (st_in == TMV_OK && (M < 0 || M > M_max)) ? TMV_ERR_INPUT : st_in;
    const uint64_t stream = (step << 32) | static_cast<uint32_t>(b);

    // outputs: slice 0 writes the path, the length and a data error; the slice holding the
    // final draw writes the token
    auto finish = [&](int code, int acc, int tok, bool mine) {
        __syncthreads();
        if (code != TMV_OK) { acc = 0; tok = 0; }
        if (k == 0)
            for (int j = tid; j < D_max; j += kSampleThreads)
                if (code != TMV_OK || j >= acc) pth[j] = 0;
        if (tid == 0) {
            if (code == TMV_ERR_DEVICE) {
                status[b] = TMV_ERR_DEVICE;
            } else if (k == 0) {
                accept_len[b] = acc;
                if (code != TMV_OK) {
                    next_token[b] = 0;
                    if (st_in == TMV_OK) status[b] = code;
                }
            }
            if (code == TMV_OK && mine) next_token[b] = tok;
        }
        seq_leave(ss, K);
    };
    if (st != TMV_OK) { finish(st, 0, 0, false); return; }

    // live tokens in range (every slice checks all of them: the same answer everywhere)
    int bad = 0;
    for (int i = tid + 1; i <= M; i += kSampleThreads)
        if (depth[static_cast<int64_t>(b) * R + i] >= 1) {
            const int t = tokens[static_cast<int64_t>(b) * R + i];
            if (t < 0 || t >= V) bad = 1;
        }
    if (block_or(bad, &L.flag)) { finish(TMV_ERR_INPUT, 0, 0, false); return; }

    // load (W, S) = quantised p row `row`, renormalised to <= 48 bits; 1 on success,
    // 0 on bad data, -1 when the other slices did not come
    auto load_p = [&](int row, Dist &Dd) -> int {
        const float *pr = p + b * psb + static_cast<int64_t>(row) * psr;
        int bd = 0;
        u128 s = 0;
        strided_pass(x_lo, x_hi, [&](int x) { return pr[x]; }, [&](int, float v) { s += quantise(v, bd); });
        SeqView v = seq_reduce(ss, K, k, phase, s, 0, 0, bd ? kFlagBad : 0, L);
        if (v.flags & kFlagTimeout) return -1;
        if ((v.flags & kFlagBad) || v.total == 0) return 0;
        Dd.row = pr; Dd.shift = 0; Dd.stored = false;
        const int bl = tmv::bitlen_u128(v.total);
        if (bl > 48) {
            Dd.shift = bl - 48;
            u128 s2 = 0;
            strided_pass(x_lo, x_hi, [&](int x) { return pr[x]; },
                         [&](int, float v2) { s2 += quantise(v2, bd) >> Dd.shift; });
            v = seq_reduce(ss, K, k, phase, s2, 0, 0, 0, L);
            if (v.flags & kFlagTimeout) return -1;
        }
        Dd.S = static_cast<uint64_t>(v.total);
        return 1;
    };

    Dist cur;
    {
        const int r = load_p(0, cur);
        if (r <= 0) { finish(r < 0 ? TMV_ERR_DEVICE : TMV_ERR_INPUT, 0, 0, false); return; }
    }
    uint64_t n = 0;           // draws consumed
    int u = 0, acc = 0;
    for (;;) {
        // children of u in ascending id: thread c-1 tests node c (one round trip), matches
        // are compacted in order with ballots
        __syncthreads();
        {
            const int c = tid + 1;
            const bool is_kid = c <= M && depth[static_cast<int64_t>(b) * R + c] >= 1 &&
                                anc[(static_cast<int64_t>(b) * R + c) * W + 1] == u;
            const uint64_t bal = __ballot(is_kid);
            const int wv = tid / kWave;
            if ((tid & (kWave - 1)) == 0) kid_count[wv] = __popcll(bal);
            __syncthreads();
            if (is_kid) {
                int before = __popcll(bal & ((1ull << (tid & (kWave - 1))) - 1));
                for (int w2 = 0; w2 < wv; ++w2) before += kid_count[w2];
                kids[before] = c;
            }
            if (tid == 0) {
                int kk = 0;
                for (int w2 = 0; w2 < kSampleWaves; ++w2) kk += kid_count[w2];
                nkids = kk;
            }
        }
        __syncthreads();
        const int nk = nkids;
        bool moved = false;
        if (nk > 0) {
            const float *qr = q + b * qsb + static_cast<int64_t>(u) * qsr;
            int bd = 0;
            u128 sq = 0;
            strided_pass(x_lo, x_hi, [&](int x) { return qr[x]; }, [&](int, float v) { sq += quantise(v, bd); });
            SeqView vq = seq_reduce(ss, K, k, phase, sq, 0, 0, bd ? kFlagBad : 0, L);
            if (vq.flags & kFlagTimeout) { finish(TMV_ERR_DEVICE, 0, 0, false); return; }
            // sum of Wq: at most V * 2^32 < 2^64
            const uint64_t SQ = static_cast<uint64_t>(vq.total);
            if ((vq.flags & kFlagBad) || SQ == 0) { finish(TMV_ERR_INPUT, 0, 0, false); return; }
            uint64_t w_next = 0;                   // W at the current child's token once W is stored
            for (int ci = 0; ci < nk; ++ci) {
                const int c = kids[ci];
                const int x = tokens[static_cast<int64_t>(b) * R + c];
                int bd2 = 0;
                const uint64_t wx = cur.stored ? w_next : quantise(cur.row[x], bd2) >> cur.shift;
                const uint64_t wqx = quantise(qr[x], bd2);
                const uint64_t U = tmv::philox_word(seed, stream, n++) >> 40;
                if (static_cast<u128>(U) * wqx * cur.S < (static_cast<u128>(wx) * SQ) << 24) {
                    if (k == 0 && tid == 0) pth[acc] = c;
                    ++acc;
                    u = c;
                    const int r = load_p(c, cur);
                    if (r <= 0) { finish(r < 0 ? TMV_ERR_DEVICE : TMV_ERR_INPUT, 0, 0, false); return; }
                    moved = true;
                    break;
                }
                // residual: W(y) <- max(0, W(y) SQ - Wq(y) S), renormalised.  The owner of the
                // next child's token publishes W there: first its current value (kept when the
                // residual is empty), then its new one.
                const int xn = ci + 1 < nk ? tokens[static_cast<int64_t>(b) * R + kids[ci + 1]] : 0;
                const int own_n = owner_of(xn);
                const bool have_xn = ci + 1 < nk && xn >= x_lo && xn < x_hi;
                auto load_pair = [&](int y) {
                    RowPair r;
                    r.a = cur.stored ? w[y] : static_cast<uint64_t>(__float_as_uint(cur.row[y]));
                    r.q = qr[y];
                    return r;
                };
                auto w_of = [&](const RowPair &r) {
                    int bd3 = 0;
                    return cur.stored ? r.a : quantise(__uint_as_float(static_cast<uint32_t>(r.a)), bd3) >> cur.shift;
                };
                uint64_t pub = 0;
                if (have_xn) {
                    int bd3 = 0;
                    pub = cur.stored ? w[xn] : quantise(cur.row[xn], bd3) >> cur.shift;
                }
                u128 sn = 0;
                strided_pass(x_lo, x_hi, load_pair, [&](int, const RowPair &r) {
                    int bd3 = 0;
                    const u128 a = static_cast<u128>(w_of(r)) * SQ;
                    const u128 c2 = static_cast<u128>(quantise(r.q, bd3)) * cur.S;
                    sn += a > c2 ? a - c2 : 0;
                });
                SeqView vs = seq_reduce(ss, K, k, phase, sn, pub, own_n, 0, L);
                if (vs.flags & kFlagTimeout) { finish(TMV_ERR_DEVICE, 0, 0, false); return; }
                if (vs.total == 0) {                // empty residual: keep the distribution
                    w_next = vs.extra;
                    continue;
                }
                const int bl = tmv::bitlen_u128(vs.total);
                const int sh = bl > 48 ? bl - 48 : 0;
                // write the shifted residual; reading W(y) and writing w[y] happen in the
                // same thread for the same y, so the update is safe in place
                u128 s2 = 0;
                uint64_t pub2 = 0;
                strided_pass(x_lo, x_hi, load_pair, [&](int y, const RowPair &r) {
                    int bd3 = 0;
                    const u128 a = static_cast<u128>(w_of(r)) * SQ;
                    const u128 c2 = static_cast<u128>(quantise(r.q, bd3)) * cur.S;
                    const uint64_t nv = static_cast<uint64_t>((a > c2 ? a - c2 : 0) >> sh);
                    w[y] = nv;
                    s2 += nv;
                    if (have_xn && y == xn) pub2 = nv;
                });
                // (the thread that wrote the token's weight holds it; pass it to the block)
                if (have_xn) {
                    __syncthreads();
                    if (tid == (xn - x_lo) % kSampleThreads) L.res[0] = pub2;
                    __syncthreads();
                    pub2 = L.res[0];
                }
                SeqView vw = seq_reduce(ss, K, k, phase, s2, pub2, own_n, 0, L);
                if (vw.flags & kFlagTimeout) { finish(TMV_ERR_DEVICE, 0, 0, false); return; }
                cur.stored = true;
                cur.S = static_cast<uint64_t>(vw.total);
                w_next = vw.extra;
            }
            if (moved) continue;
        }
        // draw the bonus (no children) or the correction (all refused) from (W, S):
        // t = floor(word_hi * S / 2^32), the token is the first x whose running sum of W
        // exceeds t.  Slice sums locate the slice; inside it, contiguous segments per thread
        // (a multiple of 4 entries) and an exclusive scan of their sums locate the token.
        const uint64_t word = tmv::philox_word(seed, stream, n++);
        const u128 t = (static_cast<u128>(word >> 32) * cur.S) >> 32;
        const int len = x_hi - x_lo;
        const int seg = ((len + kSampleThreads - 1) / kSampleThreads + 3) & ~3;
        const int s0 = min(x_hi, x_lo + tid * seg), s1 = min(x_hi, s0 + seg);
        u128 ssum = 0;
        int bd = 0;
        constexpr int kDrawBatch = 16;
        for (int xb = s0; xb < s1; xb += kDrawBatch) {
            uint64_t vals[kDrawBatch];
#pragma unroll
            for (int j = 0; j < kDrawBatch; ++j) {
                const int x = xb + j;
                vals[j] = x < s1 ? (cur.stored ? w[x] : static_cast<uint64_t>(__float_as_uint(cur.row[x]))) : 0;
            }
#pragma unroll
            for (int j = 0; j < kDrawBatch; ++j)
                if (xb + j < s1)
                    ssum += cur.stored ? vals[j] : quantise(__uint_as_float(static_cast<uint32_t>(vals[j])), bd) >> cur.shift;
        }
        // inclusive scan of the segment sums inside the wave (shuffles up, 32-bit parts)
        const int lane = tid & (kWave - 1), wv = tid / kWave;
        u128 incl = ssum;
        for (int o = 1; o < kWave; o <<= 1) {
            u128 y = 0;
#pragma unroll
            for (int part = 0; part < 4; ++part) {
                const uint32_t v32 = static_cast<uint32_t>(incl >> (32 * part));
                y |= static_cast<u128>(static_cast<uint32_t>(__shfl_up(v32, o, kWave))) << (32 * part);
            }
            if (lane >= o) incl += y;
        }
        __syncthreads();
        if (lane == kWave - 1) scan_sh[wv] = incl;
        if (tid == 0) draw_tok = -1;
        __syncthreads();
        u128 wbefore = 0;
        for (int w2 = 0; w2 < wv; ++w2) wbefore += scan_sh[w2];
        // the slice sums: the same values as S (the distribution is unchanged since)
        const SeqView vd = seq_reduce(ss, K, k, phase, ssum, 0, 0, 0, L);
        if (vd.flags & kFlagTimeout) { finish(TMV_ERR_DEVICE, 0, 0, false); return; }
        const u128 excl = vd.before + wbefore + incl - ssum;
        const bool mine = vd.before <= t && t < vd.before + vd.own;      // t lies in this slice
        // the thread whose segment holds the crossing point finds the token
        if (ssum > 0 && excl <= t && t < excl + ssum) {
            u128 cacc = excl;
            for (int x = s0; x < s1; ++x) {
                cacc += cur.stored ? w[x] : quantise(cur.row[x], bd) >> cur.shift;
                if (cacc > t) { draw_tok = x; break; }
            }
        }
        __syncthreads();
        const int tok = draw_tok >= 0 ? draw_tok : x_hi - 1;
        finish(TMV_OK, acc, tok, mine);
        return;
    }
}

}  // namespace

// sampling workspace: [B][V] u64 working distributions | [B] sequence synchronisation
// blocks (their counts zero between calls)
static size_t sample_ws_bytes(int B, int V, size_t *off_sync) {
    const size_t dist = (static_cast<size_t>(B) * V * sizeof(uint64_t) + 255) / 256 * 256;
    if (off_sync) *off_sync = dist;
    return dist + static_cast<size_t>(B) * sizeof(SeqSync);
}

// workgroups per sequence: at most one workgroup per compute unit in all (so every workgroup
// a barrier waits for is resident), at most kMaxSlices, slices of >= 1024 entries
static int sample_slices(int B, int V) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 1;
    int K = cus / (B > 0 ? B : 1);
    if (K > kMaxSlices) K = kMaxSlices;
    if (K > V / 1024) K = V / 1024;
    return K < 1 ? 1 : K;
}

extern "C" size_t tmv_tree_accept_workspace(int mode, int B, int M_max, int V)
{
    if (B <= 0 || M_max < 0 || V <= 0) return 256;
    if (mode == TMV_ACCEPT_GREEDY) {
        const int nchunk = (V + kScanChunk - 1) / kScanChunk;
        return static_cast<size_t>(B) * (M_max + 1) * nchunk * sizeof(uint64_t) + 256;
    }
    return sample_ws_bytes(B, V, nullptr);
}

extern "C" int tmv_tree_accept(int mode, int B, int M_max, int D_max, int V,
                               const int32_t *tokens, int row_dtype, const void *teacher,
                               int64_t t_stride_b, int64_t t_stride_row,
                               const float *draft_q, int64_t q_stride_b, int64_t q_stride_row,
                               uint64_t seed, uint64_t step,
                               const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                               int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token,
                               void *workspace, size_t workspace_bytes, void *stream)
{
    if (mode != TMV_ACCEPT_GREEDY && mode != TMV_ACCEPT_SAMPLE) return TMV_ERR_ARG;
    if (B < 0 || M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128 || V < 1) return TMV_ERR_ARG;
    if (t_stride_b < 0 || t_stride_row < 0) return TMV_ERR_ARG;
    if (B == 0) return TMV_OK;
    if (!tokens || !teacher || !n_nodes || !anc || !depth || !status || !accept_len || !next_token)
        return TMV_ERR_ARG;
    if (D_max > 0 && !path) return TMV_ERR_ARG;
    if (!workspace || workspace_bytes < tmv_tree_accept_workspace(mode, B, M_max, V)) return TMV_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(workspace) & 15u) != 0) return TMV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);

    if (mode == TMV_ACCEPT_GREEDY) {
        if (row_dtype != TMV_F32 && row_dtype != TMV_BF16) return TMV_ERR_ARG;
        const int nchunk = (V + kScanChunk - 1) / kScanChunk;
        const int64_t blocks = static_cast<int64_t>(B) * (M_max + 1) * nchunk;
        if (blocks > 0x7fffffff) return TMV_ERR_ARG;
        uint64_t *keys = reinterpret_cast<uint64_t *>(ws);
        if (row_dtype == TMV_F32)
            hipLaunchKernelGGL(greedy_scan_kernel<TMV_F32>, dim3(static_cast<unsigned>(blocks)), dim3(kScanThreads), 0, s,
                               M_max, V, nchunk, teacher, t_stride_b, t_stride_row, n_nodes, depth, status, keys);
        else
            hipLaunchKernelGGL(greedy_scan_kernel<TMV_BF16>, dim3(static_cast<unsigned>(blocks)), dim3(kScanThreads), 0, s,
                               M_max, V, nchunk, teacher, t_stride_b, t_stride_row, n_nodes, depth, status, keys);
        hipLaunchKernelGGL(greedy_select_kernel, dim3(B), dim3(kScanThreads), 0, s, M_max, D_max, V, nchunk, tokens,
                           n_nodes, anc, depth, status, accept_len, path, next_token, keys);
        return tmv_host::launch_status(hipGetLastError());
    }
    if (row_dtype != TMV_F32 || !draft_q || q_stride_b < 0 || q_stride_row < 0) return TMV_ERR_ARG;
    const int K = sample_slices(B, V);
    size_t off_sync = 0;
    sample_ws_bytes(B, V, &off_sync);
    hipLaunchKernelGGL(sample_walk_kernel, dim3(static_cast<unsigned>(B) * K), dim3(kSampleThreads), 0, s, M_max,
                       D_max, V, K, tokens, static_cast<const float *>(teacher), t_stride_b, t_stride_row, draft_q,
                       q_stride_b, q_stride_row, seed, step, n_nodes, anc, depth, status, accept_len, path,
                       next_token, reinterpret_cast<uint64_t *>(ws), reinterpret_cast<SeqSync *>(ws + off_sync));
    return tmv_host::launch_status(hipGetLastError());
}
