// accept.hip -- choosing the accepted path of a verified draft tree (gfx950).
//
// GREEDY: the teacher's argmax of every live row, then the deepest node whose whole
//   path matches those choices (Medusa section of "Speculative Decoding Hierarquico":
//   the longest valid branch is kept).  The row scans are the HBM-bound part: one
//   workgroup per (sequence, row, vocabulary chunk) reads its chunk with 16-byte loads
//   and reduces it to a 64-bit key (order-preserving value bits << 32 | ~index, -0 keyed
//   as +0), so max() gives the largest value and, on ties, the smallest index.  When the
//   whole scan is resident on the device at once, the keys meet in one 64-bit device-scope
//   atomic maximum per row, the last chunk of a row to arrive counts the row in for its
//   sequence, and the last row of a sequence chooses the path in the same launch (counters
//   only: no workgroup ever waits for another).  Larger scans write one key per chunk and
//   a second kernel (one workgroup per sequence, ordered after the scan on the stream)
//   merges them and picks the path: there the per-workgroup atomics would lengthen every
//   round of resident workgroups.
// SAMPLE: modified rejection sampling (same page, its rejection-sampling section and
//   FAQ), children of the current node tried in ascending id against the running
//   residual, which against one draft row keeps the form (p - c q)+.  Exact integer fixed
//   point, so the result is bit-identical to any correct implementation.  K workgroups
//   walk a sequence, one per vocabulary slice, holding their slices of the node's two rows
//   in registers; every refusal is one exact sum over them, met at a bounded barrier.
#include <mutex>

#include "tmv_device.hpp"

namespace {

using tmv::kWave;
using tmv::u128;

// ============================================================== greedy
constexpr int kScanThreads = 256;
constexpr int kScanChunk = 4096;          // vocabulary entries per workgroup (four 16-byte fp32 loads per thread)
constexpr uint64_t kNanKey = ~0ull;       // a chunk with a NaN reports the all-ones key
constexpr int kSelectBatch = 8;           // chunk keys per thread in flight in the path choice
// greedy workspace: [one-launch part: per (sequence, row) a 64-bit key and an arrival
// counter, per sequence an arrival counter, each on a 128-byte line of its own (atomics
// on one line serialise); zero between calls] [two-launch part: the chunk keys]
constexpr int kSlot = 128;

__device__ __forceinline__ uint32_t order_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// key of value v at index idx: order-preserving value bits << 32 | ~idx, with -0 keyed as
// +0 (the two compare equal, so the smaller index wins between them)
__device__ __forceinline__ uint64_t value_key(float v, int idx) {
    if (__float_as_uint(v) == 0x80000000u) v = 0.0f;
    return (static_cast<uint64_t>(order_bits(v)) << 32) | (0xffffffffu - static_cast<uint32_t>(idx));
}

__device__ __forceinline__ void scan_one(float v, int idx, uint64_t &best, bool &nan) {
    if (v != v) nan = true;
    const uint64_t key = value_key(v, idx);
    best = key > best ? key : best;
}

// The path choice of sequence b (one workgroup of kScanThreads threads, rows on threads):
// t(u) of every live row from its merged key, the draft tokens checked against them, the
// deepest matching node (smallest id on ties) and its path.  load_path_inputs issues the
// per-row reads (token, depth, first ancestor entries; indices clamped into the tables) so
// that they travel together with the caller's key reads; choose_path_from takes this
// thread's row key (all ones after a NaN) and does the rest.  row_argmax, if not null,
// receives t(u) of every live row and -1 elsewhere.
constexpr int kAncBatch = 8;                       // ancestor entries per node fetched at once

struct PathInputs {
    int M, st_in, tok, dep;
    int a8[kAncBatch];
    const int32_t *arow;
};

__device__ __forceinline__ PathInputs load_path_inputs(int b, int M_max, int D_max, const int32_t *__restrict__ tokens,
                                                       const int32_t *__restrict__ n_nodes,
                                                       const int32_t *__restrict__ anc,
                                                       const int32_t *__restrict__ depth,
                                                       const int32_t *__restrict__ status)
{
    PathInputs in;
    const int R = M_max + 1, W = D_max + 1, tid = threadIdx.x;
    const int row = tid < R ? tid : R - 1;
    const int64_t rb = static_cast<int64_t>(b) * R + row;
    in.M = n_nodes[b];
    in.st_in = status[b];
    in.tok = tokens[rb];
    in.dep = row > 0 ? depth[rb] : 0;
    in.arow = anc + rb * W;
#pragma unroll
    for (int k = 0; k < kAncBatch; ++k) in.a8[k] = in.arow[k < W ? k : W - 1];
    return in;
}

__device__ __forceinline__ void choose_path_from(const PathInputs &in, int b, int M_max, int D_max, int V,
                                                 uint64_t krow, int32_t *__restrict__ status,
                                                 int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                                                 int32_t *__restrict__ next_token, const int32_t *__restrict__ anc,
                                                 int32_t *__restrict__ row_argmax)
{
    __shared__ int32_t tsel[129];
    __shared__ int32_t anc_sh[129][kAncBatch];     // every row's first ancestor entries
    __shared__ uint64_t match_w[3];                // bit u: node u's token is its parent row's choice
    __shared__ int bad;
    __shared__ uint32_t best;
    const int R = M_max + 1, W = D_max + 1;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int M = in.M, st_in = in.st_in, tok = in.tok, dep = in.dep;
    const int32_t *arow = in.arow;
    const int64_t rb = static_cast<int64_t>(b) * R + (tid < R ? tid : R - 1);

    // a node count outside [0, M_max] cannot come with an OK status from the build stage;
    // it is rejected here so that no row beyond the tables is ever addressed
    const int st = (st_in == TMV_OK && (M < 0 || M > M_max)) ? TMV_ERR_INPUT : st_in;
    int32_t *pth = path + static_cast<int64_t>(b) * D_max;
    if (tid == 0) {
        bad = st != TMV_OK;
        best = 0u;
    }
    if (tid < R) {
#pragma unroll
        for (int k = 0; k < kAncBatch; ++k) anc_sh[tid][k] = in.a8[k];
    }
    __syncthreads();
    const bool row_live = st == TMV_OK && tid < R && tid <= M && (tid == 0 || dep >= 1);
    if (row_live) {
        if (krow == kNanKey) bad = 1;
        tsel[tid] = static_cast<int32_t>(0xffffffffu - static_cast<uint32_t>(krow & 0xffffffffu));
        if (tid > 0 && (tok < 0 || tok >= V)) bad = 1;
    }
    __syncthreads();
    if (row_argmax && tid < R) row_argmax[rb] = (bad || !row_live) ? -1 : tsel[tid];
    if (bad) {
        for (int j = tid; j < D_max; j += kScanThreads) pth[j] = 0;
        if (tid == 0) {
            accept_len[b] = 0;
            next_token[b] = 0;
            if (st_in == TMV_OK) status[b] = TMV_ERR_INPUT;
        }
        return;
    }
    // node u (live, depth >= 1) matches its parent row when its token is that row's choice;
    // anc[u][1] is the parent (0: the root).  One ballot word per wave of rows.
    const bool node = tid >= 1 && tid <= M && dep >= 1;
    const bool m = node && tok == tsel[node ? in.a8[1] : 0];
    const uint64_t bal = __builtin_amdgcn_ballot_w64(m);
    if (lane == 0 && wv < 3) match_w[wv] = bal;
    __syncthreads();
    // node u is accepted iff every node on its path matches (the path is u's ancestor-or-self
    // row up to its depth); the chosen node maximises (depth, -id): key = depth << 8 | (255 - id)
    if (node) {
        const uint64_t w0 = match_w[0], w1 = match_w[1], w2 = match_w[2];
        auto bit = [&](int a) {
            const uint64_t w = a < 64 ? w0 : a < 128 ? w1 : w2;
            return ((w >> (a & 63)) & 1ull) != 0;
        };
        bool ok = true;
#pragma unroll
        for (int k = 0; k < kAncBatch; ++k)
            if (k < dep) ok = ok & bit(in.a8[k]);
        for (int k = kAncBatch; k < dep && ok; ++k) ok = bit(arow[k]);
        if (ok) atomicMax(&best, (static_cast<uint32_t>(dep) << 8) | static_cast<uint32_t>(255 - tid));
    }
    __syncthreads();
    const uint32_t kb = best;
    const int star = kb ? 255 - static_cast<int>(kb & 255u) : 0;
    const int dstar = static_cast<int>(kb >> 8);
    if (tid == 0) {
        accept_len[b] = dstar;
        next_token[b] = tsel[star];
    }
    // the path root -> leaf is the chosen node's ancestor row read backwards; its first
    // kAncBatch entries are already in LDS
    for (int j = tid; j < D_max; j += kScanThreads) {
        const int e = dstar - 1 - j;
        pth[j] = j >= dstar ? 0 : e < kAncBatch ? anc_sh[star][e] : anc[(static_cast<int64_t>(b) * R + star) * W + e];
    }
}

// The 64-bit key of chunk `chunk` of row u of sequence b (kScanChunk entries), returned to
// thread 0.  In a whole, aligned chunk each thread's values are reduced in ascending index
// order by a running maximum under a strict comparison (the first of equal values is kept,
// -0 equals +0, NaN fails every comparison and is flagged on its own) and the key is formed
// once per thread; the all-ones key reports a NaN.
template <int DT>
__device__ __forceinline__ uint64_t chunk_key(int V, const void *__restrict__ teacher, int64_t sb, int64_t sr, int b,
                                              int u, int chunk)
{
    __shared__ uint64_t red[kScanThreads / kWave];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    constexpr int kElem = DT == TMV_F32 ? 4 : 2;
    const int x0 = chunk * kScanChunk;
    const int x1 = min(V, x0 + kScanChunk);
    const char *row = static_cast<const char *>(teacher) + (b * sb + static_cast<int64_t>(u) * sr) * kElem;
    uint64_t best = 0;
    bool nan = false;
    if (x1 - x0 == kScanChunk && ((reinterpret_cast<uintptr_t>(row + x0 * kElem) & 15u) == 0)) {
        constexpr int kPer = kScanChunk * kElem / (16 * kScanThreads);      // 16-byte loads per thread
        constexpr int kPerLoad = 16 / kElem;                                 // values per load
        // (the logits are read once: non-temporal loads stream them past the caches -- workload
        // 3's scan 116 -> 99 us, workload 2's 12.2 -> 11.2 us)
        typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
        const u32x4_nt *r16 = reinterpret_cast<const u32x4_nt *>(row + x0 * kElem);
        uint4 h[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const u32x4_nt v = __builtin_nontemporal_load(r16 + tid + i * kScanThreads);
            h[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
        auto val = [&](int k) -> float {
            const uint4 &q = h[k / kPerLoad];
            const int e = k % kPerLoad, wi = e / (kPerLoad / 4);
            const uint32_t w = wi == 0 ? q.x : wi == 1 ? q.y : wi == 2 ? q.z : q.w;
            if constexpr (DT == TMV_F32) return __uint_as_float(w);
            else return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
        };
        float m = val(0);
        int g = 0;
        nan = m != m;
#pragma unroll
        for (int k = 1; k < kPer * kPerLoad; ++k) {
            const float v = val(k);
            nan = nan || v != v;
            const bool c = v > m;
            m = c ? v : m;
            g = c ? k : g;
        }
        best = value_key(m, x0 + kPerLoad * (tid + (g / kPerLoad) * kScanThreads) + g % kPerLoad);
    } else if constexpr (DT == TMV_F32) {
        const float *r = reinterpret_cast<const float *>(row);
        for (int x = x0 + tid; x < x1; x += kScanThreads) scan_one(r[x], x, best, nan);
    } else {
        const uint16_t *r = reinterpret_cast<const uint16_t *>(row);
        for (int x = x0 + tid; x < x1; x += kScanThreads) scan_one(tmv::bf16_to_f32(r[x]), x, best, nan);
    }
    if (nan) best = kNanKey;
    best = tmv::wave_max_u64(best);
    if (lane == 0) red[wv] = best;
    __syncthreads();
    uint64_t k = red[0];
    for (int w = 1; w < kScanThreads / kWave; ++w) k = red[w] > k ? red[w] : k;
    return k;
}

// Two launches, first: one workgroup per (sequence, row, chunk of kScanChunk entries) writes
// the chunk's key.  The liveness words (status, n_nodes, the row's depth) are read first and
// a dead row loads nothing of its logits.
template <int DT>
__global__ void __launch_bounds__(kScanThreads)
greedy_scan_kernel(int M_max, int V, int nchunk, const void *__restrict__ teacher, int64_t sb, int64_t sr,
                   const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ depth,
                   const int32_t *__restrict__ status, uint64_t *__restrict__ keys)
{
    const int R = M_max + 1;
    const int chunk = blockIdx.x % nchunk;
    const int u = (blockIdx.x / nchunk) % R;
    const int b = blockIdx.x / (nchunk * R);
    const int M = n_nodes[b];
    const int st = status[b];
    const int dp = u > 0 ? depth[static_cast<int64_t>(b) * R + u] : 1;
    if (st != TMV_OK || M < 0 || M > M_max || u > M || dp < 1) return;
    const uint64_t k = chunk_key<DT>(V, teacher, sb, sr, b, u, chunk);
    if (threadIdx.x == 0) keys[(static_cast<int64_t>(b) * R + u) * nchunk + chunk] = k;
}

// Two launches, second: one workgroup per sequence, after the scan: the chunk keys of the sequence ([row][chunk],
// contiguous) are read by all threads in coalesced batches, issued together with the
// per-row reads of the path choice, and merged per row with LDS atomics; then the path is
// chosen.  Keys of rows beyond n_nodes were not written in this call and are not read;
// those of other dead rows may be stale and are never used.
__global__ void __launch_bounds__(kScanThreads)
greedy_select_kernel(int M_max, int D_max, int V, int nchunk, const int32_t *__restrict__ tokens,
                     const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ anc,
                     const int32_t *__restrict__ depth, int32_t *__restrict__ status,
                     int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                     int32_t *__restrict__ next_token, const uint64_t *__restrict__ keys)
{
    __shared__ unsigned long long rowkey[129];
    const int R = M_max + 1, b = blockIdx.x, tid = threadIdx.x;
    const int n = R * nchunk;                          // < 2^27: R <= 129, nchunk < 2^19
    const uint64_t *kb = keys + static_cast<int64_t>(b) * n;
    if (tid < R) rowkey[tid] = 0;
    const PathInputs in = load_path_inputs(b, M_max, D_max, tokens, n_nodes, anc, depth, status);
    const int M = in.M;
    __syncthreads();
    // key k = row * nchunk + chunk; this thread visits k = tid, tid + 256, ... and carries
    // (row, chunk) along instead of dividing
    int row = tid / nchunk, c = tid - row * nchunk;
    const int drow = kScanThreads / nchunk, dc = kScanThreads - drow * nchunk;
    for (int k0 = 0; k0 < n; k0 += kScanThreads * kSelectBatch) {
        uint64_t kv[kSelectBatch];
        int rw[kSelectBatch];
#pragma unroll
        for (int j = 0; j < kSelectBatch; ++j) {
            const int k = k0 + tid + j * kScanThreads;
            rw[j] = row;
            kv[j] = k < n && row <= M ? kb[k] : 0;
            row += drow;
            c += dc;
            if (c >= nchunk) {
                c -= nchunk;
                ++row;
            }
        }
#pragma unroll
        for (int j = 0; j < kSelectBatch; ++j)
            if (kv[j] != 0) atomicMax(&rowkey[rw[j]], static_cast<unsigned long long>(kv[j]));
    }
    __syncthreads();
    choose_path_from(in, b, M_max, D_max, V, rowkey[tid < R ? tid : 0], status, accept_len, path, next_token, anc,
                     static_cast<int32_t *>(nullptr));
}

// The greedy accept in one launch (the whole grid resident at once): one workgroup per
// (sequence, row, chunk), liveness as in greedy_scan_kernel.  Then:
//   * the chunk's key goes into the row's key by a device-scope atomic maximum, and once
//     that has completed the workgroup counts itself in on the row's counter;
//   * the last chunk of a live row to arrive (and chunk 0 of a dead row, at once) counts
//     the row in on the sequence's counter;
//   * the last row of the sequence to arrive reads every row key with agent-coherent loads
//     and chooses the path.
// Every counter is reset by the workgroup that completes it and every row key by the
// chooser, so a zero-filled workspace is left zero by each call.
template <int DT>
__global__ void __launch_bounds__(kScanThreads)
greedy_accept_kernel(int M_max, int D_max, int V, int nchunk, const void *__restrict__ teacher, int64_t sb,
                     int64_t sr, const int32_t *__restrict__ tokens, const int32_t *__restrict__ n_nodes,
                     const int32_t *__restrict__ anc, const int32_t *__restrict__ depth,
                     int32_t *__restrict__ status, int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                     int32_t *__restrict__ next_token, char *__restrict__ ws)
{
    __shared__ int s_flag;
    const int R = M_max + 1;
    const int chunk = blockIdx.x % nchunk;
    const int u = (blockIdx.x / nchunk) % R;
    const int b = blockIdx.x / (nchunk * R);
    const int tid = threadIdx.x;
    const int B = gridDim.x / (nchunk * R);
    unsigned long long *row_key = reinterpret_cast<unsigned long long *>(ws + (static_cast<int64_t>(b) * R + u) * kSlot);
    int32_t *row_cnt = reinterpret_cast<int32_t *>(ws + (static_cast<int64_t>(B) * R + static_cast<int64_t>(b) * R + u) * kSlot);
    int32_t *seq_cnt = reinterpret_cast<int32_t *>(ws + (2 * static_cast<int64_t>(B) * R + b) * kSlot);
    const int M = n_nodes[b];
    const int st = status[b];
    const int dp = u > 0 ? depth[static_cast<int64_t>(b) * R + u] : 1;
    const bool live = st == TMV_OK && M >= 0 && M <= M_max && u <= M && dp >= 1;
    if (!live && chunk != 0) return;

    if (live) {
        const uint64_t k = chunk_key<DT>(V, teacher, sb, sr, b, u, chunk);
        if (tid == 0) {
            // the maximum has been performed (its old value has returned, the returning form)
            // before the arrival is counted, so the row's last arrival finds every chunk's key
            // in the row key
            const unsigned long long old_k = __hip_atomic_fetch_max(row_key, static_cast<unsigned long long>(k),
                                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            asm volatile("" ::"v"(old_k));
            const int old = __hip_atomic_fetch_add(row_cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old == nchunk - 1;
            if (last) __hip_atomic_store(row_cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_flag = last ? 1 : 0;
        }
        __syncthreads();
        if (s_flag == 0) return;
    }
    // this row is complete (or dead): count it in for the sequence; the last row chooses.
    // (Only the chooser reads the path inputs, together with the row keys: issued before the
    // arrival they would hold its result back, loads completing in issue order.)
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(seq_cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old == R - 1;
        if (last) __hip_atomic_store(seq_cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_flag = last ? 2 : 0;
    }
    __syncthreads();
    if (s_flag != 2) return;
    // every row of the sequence has arrived: its keys are final (dead rows' stay zero)
    const PathInputs in = load_path_inputs(b, M_max, D_max, tokens, n_nodes, anc, depth, status);
    uint64_t krow = 0;
    if (tid < R) {
        unsigned long long *rk = reinterpret_cast<unsigned long long *>(ws + (static_cast<int64_t>(b) * R + tid) * kSlot);
        krow = __hip_atomic_load(rk, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(rk, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    choose_path_from(in, b, M_max, D_max, V, krow, status, accept_len, path, next_token, anc,
                     static_cast<int32_t *>(nullptr));
}

// The LM-head path's choice (one workgroup per sequence, ordered after the LM-head kernel
// on the stream, which merged one key per row with atomics): each row's key is read once
// and set back to zero for the next call.
__global__ void __launch_bounds__(kScanThreads)
lm_select_kernel(int M_max, int D_max, int V, const int32_t *__restrict__ tokens, const int32_t *__restrict__ n_nodes,
                 const int32_t *__restrict__ anc, const int32_t *__restrict__ depth, int32_t *__restrict__ status,
                 int32_t *__restrict__ accept_len, int32_t *__restrict__ path, int32_t *__restrict__ next_token,
                 uint64_t *__restrict__ keys, int32_t *__restrict__ row_argmax)
{
    const int b = blockIdx.x, R = M_max + 1, tid = threadIdx.x;
    const int64_t rb = static_cast<int64_t>(b) * R + (tid < R ? tid : R - 1);
    const PathInputs in = load_path_inputs(b, M_max, D_max, tokens, n_nodes, anc, depth, status);
    const uint64_t krow = keys[rb];
    if (tid < R) keys[rb] = 0;
    choose_path_from(in, b, M_max, D_max, V, krow, status, accept_len, path, next_token, anc, row_argmax);
}

// ============================================================== greedy on LM-head logits
// The teacher's logits of row u are h_u W^T: its final hidden state h_u (K entries) against
// the LM head W [V][K] (roofline section of "Speculative Decoding Hierarquico": decode
// streams the LM-head weights once per step).  Only each row's argmax is needed, so the
// logits are reduced to the greedy keys as the MFMA tiles produce them and never written:
// per step that saves writing and re-reading rows x V fp32 logits, and the weights -- the
// whole cost at a few dozen rows -- are read once.
//   * a workgroup of 8 waves owns a block of 64 rows and kLmTpw vocabulary tiles of 256
//     entries; wave w computes entries 32w .. +32 of each tile (two 16-entry MFMA row tiles)
//     against the 64 rows (four 16-row column tiles), v_mfma_f32_16x16x32_bf16 over K in
//     32-wide steps;
//   * the rows' hidden states are staged in LDS one 512-wide k-block at a time (16-byte
//     pieces XOR-swizzled by row, so the operand reads of a wave hit distinct banks) and
//     shared by the waves and the tiles; the weights stream from HBM straight into
//     registers, kLmDepth steps ahead, through a fully unrolled step sequence so that every
//     step waits for exactly its own loads;
//   * each lane keeps, per row, the best (value, ~index) key; the keys are reduced over
//     the lanes and waves of the workgroup and merged into the row's key in the workspace
//     with one device-scope 64-bit atomic max per row, which the select kernel reads (and
//     clears).  A NaN logit makes the row's key all ones.
constexpr int kLmWaves = 8;
constexpr int kLmThreads = kLmWaves * kWave;
constexpr int kLmRows = 64;                            // rows per row block
constexpr int kLmVocabPerWave = 32;
constexpr int kLmTile = kLmWaves * kLmVocabPerWave;    // vocabulary entries per tile
constexpr int kLmTpw = 2;                              // tiles per workgroup
constexpr int kLmKB = 512;                             // k entries per staged block
constexpr int kLmPieces = kLmKB / 8;                   // 16-byte pieces per staged row
constexpr int kLmDepth = 8;                            // weight steps in flight per wave
constexpr int kLmBufferFlags = 0x00020000;             // raw buffer descriptor word 3 (gfx9 family)

typedef __bf16 lm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lm_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned lm_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool lm_row_live(int gr, int R, int M_max, const int32_t *__restrict__ n_nodes,
                                            const int32_t *__restrict__ depth, const int32_t *__restrict__ status)
{
    const int b = gr / R, u = gr - b * R;
    const int M = n_nodes[b];
    return status[b] == TMV_OK && M >= 0 && M <= M_max && u <= M && (u == 0 || depth[gr] >= 1);
}

// NKS = K / 32 steps (K a multiple of kLmKB), unrolled completely
template <int NKS>
__global__ void __launch_bounds__(kLmThreads)
lm_head_argmax_kernel(int B, int M_max, int V, const uint16_t *__restrict__ hidden, int64_t hsb, int64_t hsr,
                      uint32_t h_bytes, const uint16_t *__restrict__ w, int64_t wsr, uint32_t w_bytes,
                      const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ depth,
                      const int32_t *__restrict__ status, uint64_t *__restrict__ row_keys, int ntiles, int ntp,
                      int nrb)
{
    static_assert(NKS % (kLmKB / 32) == 0, "whole staged blocks");
    constexpr int kStepsPerBlock = kLmKB / 32;
    constexpr int kSteps = kLmTpw * NKS;                       // (block, tile, step) sequence
    __shared__ lm_u32x4 h_lds[kLmRows][kLmPieces];
    __shared__ uint64_t s_key[kLmWaves][kLmRows];
    __shared__ int s_any;
    const int R = M_max + 1, nrows = B * R;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c16 = lane & 15, G = lane >> 4;
    // workgroup id = XCD slot + 8 (row block + nrb * s), covering tile pair s * 8 + slot: the
    // row blocks of one tile pair share an id mod 8, hence one XCD, and are dispatched one
    // after another, so they stream the same weight rows at about the same time -- the
    // weights come from HBM once and the other row blocks read them from that XCD's L2
    const int xslot = blockIdx.x & 7, rest = blockIdx.x >> 3;
    const int tpi = (rest / nrb) * 8 + xslot;
    if (tpi >= ntp) return;
    const int rb0 = (rest % nrb) * kLmRows;

    // a row block without a live row does nothing
    if (threadIdx.x == 0) s_any = 0;
    __syncthreads();
    if (threadIdx.x < kLmRows && rb0 + static_cast<int>(threadIdx.x) < nrows &&
        lm_row_live(rb0 + threadIdx.x, R, M_max, n_nodes, depth, status))
        s_any = 1;
    __syncthreads();
    if (!s_any) return;

    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(hidden), 0,
                                                                        static_cast<int>(h_bytes), kLmBufferFlags);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(w), 0,
                                                                        static_cast<int>(w_bytes), kLmBufferFlags);
    // staging of a k-block: thread t moves pieces t + 512 i (row q / kLmPieces, piece
    // q % kLmPieces) of the block; rows past the tensor are clamped (never merged)
    constexpr int kStage = kLmRows * kLmPieces / kLmThreads;
    uint32_t soff[kStage];
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
        const int q = threadIdx.x + i * kLmThreads, r = q / kLmPieces, pc = q % kLmPieces;
        int gr = rb0 + r;
        if (gr > nrows - 1) gr = nrows - 1;
        const int b = gr / R, u = gr - b * R;
        soff[i] = static_cast<uint32_t>((b * hsb + u * hsr) * 2 + pc * 16);
    }
    // tiles of this workgroup; a missing second tile computes on clamped rows and is ignored
    int vbase[kLmTpw];
    bool tile_ok[kLmTpw];
    uint32_t woff[kLmTpw][2];
#pragma unroll
    for (int tp = 0; tp < kLmTpw; ++tp) {
        const int t = tpi + tp * ntp;
        tile_ok[tp] = t < ntiles;
        vbase[tp] = t * kLmTile + wave * kLmVocabPerWave;
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) {
            int v = vbase[tp] + vt * 16 + c16;
            if (v > V - 1) v = V - 1;
            woff[tp][vt] = static_cast<uint32_t>(v * wsr * 2 + G * 16);
        }
    }
    lm_f32x4 acc[kLmTpw][2][4];
#pragma unroll
    for (int tp = 0; tp < kLmTpw; ++tp)
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) acc[tp][vt][rt] = lm_f32x4{0.f, 0.f, 0.f, 0.f};

    // step i of the sequence: block i / (kLmTpw * kStepsPerBlock), tile (i / kStepsPerBlock)
    // % kLmTpw, k-step within the block i % kStepsPerBlock
    // (k offsets go in the scalar offset operand: uniform, and no per-step address registers)
    lm_u32x4 wa[kLmDepth][2];
    auto load_w = [&](int i) {
        const int blk = i / (kLmTpw * kStepsPerBlock), tp = (i / kStepsPerBlock) % kLmTpw;
        const int ks = blk * kStepsPerBlock + i % kStepsPerBlock;
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
            wa[i % kLmDepth][vt] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[tp][vt], ks * 64, 0);
    };
    // the hidden states of block 0 go out first; each block's arrive a block ahead of use
    constexpr int kBlocks = NKS / kStepsPerBlock;
    lm_u32x4 hv[kStage];
#pragma unroll
    for (int j = 0; j < kStage; ++j) hv[j] = __builtin_amdgcn_raw_buffer_load_b128(hr, soff[j], 0, 0);
#pragma unroll
    for (int i = 0; i < kLmDepth; ++i) load_w(i);
    // B operand of row rt*16 + c16 at k-step ks of the staged block: piece 4 ks + G
    auto h_frag = [&](int rt, int ks) {
        const int r = rt * 16 + c16;
        return h_lds[r][(ks * 4 + G) ^ (r & 15)];
    };
#pragma unroll
    for (int i = 0; i < kSteps; ++i) {
        const int blk = i / (kLmTpw * kStepsPerBlock), tp = (i / kStepsPerBlock) % kLmTpw;
        const int ks = i % kStepsPerBlock;
        if (i % (kLmTpw * kStepsPerBlock) == 0) {
            // stage block blk of the rows' hidden states (after every wave is done with the
            // last), then send for block blk + 1
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kStage; ++j) {
                const int q = threadIdx.x + j * kLmThreads, r = q / kLmPieces, pc = q % kLmPieces;
                h_lds[r][pc ^ (r & 15)] = hv[j];
            }
            __syncthreads();
            if (blk + 1 < kBlocks) {
#pragma unroll
                for (int j = 0; j < kStage; ++j)
                    hv[j] = __builtin_amdgcn_raw_buffer_load_b128(hr, soff[j], (blk + 1) * kLmKB * 2, 0);
            }
        }
        lm_u32x4 hb[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) hb[rt] = h_frag(rt, ks);
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
                acc[tp][vt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(lm_bf16x8, wa[i % kLmDepth][vt]), __builtin_bit_cast(lm_bf16x8, hb[rt]),
                    acc[tp][vt][rt], 0, 0, 0);
        if (i + kLmDepth < kSteps) load_w(i + kLmDepth);
        // pin the schedule: without this the scheduler sinks every load next to its use
        // (to save registers) and the steps wait for their loads one by one
        __builtin_amdgcn_sched_barrier(0);
    }
    // lane holds row rt*16 + c16 at entries vbase + vt*16 + G*4 + i
    uint64_t best[4] = {0, 0, 0, 0};
    bool nan[4] = {false, false, false, false};
#pragma unroll
    for (int tp = 0; tp < kLmTpw; ++tp) {
        if (!tile_ok[tp]) continue;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int vt = 0; vt < 2; ++vt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = vbase[tp] + vt * 16 + G * 4 + i;
                    if (v < V) scan_one(acc[tp][vt][rt][i], v, best[rt], nan[rt]);
                }
    }
    // reduce over the four lanes of a row, then over the waves, and merge into the row's key
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        uint64_t k = nan[rt] ? kNanKey : best[rt];
        uint64_t o = tmv::shfl_xor_u64(k, 16);
        k = o > k ? o : k;
        o = tmv::shfl_xor_u64(k, 32);
        k = o > k ? o : k;
        if (G == 0) s_key[wave][rt * 16 + c16] = k;
    }
    __syncthreads();
    if (threadIdx.x < kLmRows) {
        const int gr = rb0 + threadIdx.x;
        uint64_t k = s_key[0][threadIdx.x];
#pragma unroll
        for (int w2 = 1; w2 < kLmWaves; ++w2) k = s_key[w2][threadIdx.x] > k ? s_key[w2][threadIdx.x] : k;
        if (gr < nrows && lm_row_live(gr, R, M_max, n_nodes, depth, status))
            __hip_atomic_fetch_max(reinterpret_cast<unsigned long long *>(row_keys + gr),
                                   static_cast<unsigned long long>(k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// The LM-head product for more rows than one 64-row block (several sequences' trees, or
// deep trees): a block of up to 272 rows (17 row tiles of 16) against one vocabulary tile
// of 128 entries per workgroup, so that the weights are read once for all those rows (the
// 64-row kernel would stream them once per row block).  4 waves, one per SIMD (the 17 x 2
// accumulator tiles take 136 registers per lane); wave w computes entries 32w .. +32 of the
// tile, v_mfma_f32_16x16x32_bf16 over K in 32-wide steps.
//   * the rows' hidden states are staged in LDS one 128-wide k-block at a time (16-byte
//     pieces XOR-swizzled by row), the next block travelling in registers meanwhile;
//   * the weights stream from HBM straight into registers kLwDepth steps ahead, in a loop
//     whose body covers two k-blocks (kLwDepth steps, so every ring slot is a constant);
//   * the keys are formed and merged as in the 64-row kernel: per lane and row the best
//     (value, ~index), reduced over lanes and waves, one device-scope atomic max per row.
constexpr int kLwWaves = 8;
constexpr int kLwThreads = kLwWaves * kWave;
constexpr int kLwRT = 17;                              // row tiles of 16 per row block
constexpr int kLwRows = kLwRT * 16;                    // 272 rows per row block
constexpr int kLwTile = kLwWaves * kLmVocabPerWave;    // 128 vocabulary entries per workgroup
constexpr int kLwKB = 128;                             // k entries per staged block
constexpr int kLwPieces = kLwKB / 8;                   // 16-byte pieces per staged row (16)
constexpr int kLwSteps = kLwKB / 32;                   // MFMA k-steps per staged block
constexpr int kLwBody = 1;                             // staged blocks per loop iteration
constexpr int kLwDepth = kLwBody * kLwSteps;           // weight steps in flight per wave
constexpr int kLwPre = 4;                              // B-operand LDS reads in flight per wave
constexpr int kLwPiecesAll = kLwRows * kLwPieces;
constexpr int kLwStage = (kLwPiecesAll + kLwThreads - 1) / kLwThreads;   // staged pieces per thread (9)
static_assert(kLwPieces == 16, "the row swizzle spans 16 pieces");

__global__ void __launch_bounds__(kLwThreads)
lm_head_argmax_wide_kernel(int B, int M_max, int K, int V, const uint16_t *__restrict__ hidden, int64_t hsb,
                           int64_t hsr, uint32_t h_bytes, const uint16_t *__restrict__ w, int64_t wsr,
                           uint32_t w_bytes, const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ depth,
                           const int32_t *__restrict__ status, uint64_t *__restrict__ row_keys, int ntiles, int nrb)
{
    __shared__ lm_u32x4 h_lds[kLwRows][kLwPieces];
    __shared__ uint64_t s_key[kLwWaves][kLwRows];
    __shared__ int s_any;
    const int R = M_max + 1, nrows = B * R;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int c16 = lane & 15, G = lane >> 4;
    // workgroup id = XCD slot + 8 (row block + nrb * s), covering tile s * 8 + slot: the row
    // blocks of one tile share an XCD and are dispatched one after another (as in the
    // 64-row kernel)
    const int xslot = blockIdx.x & 7, rest = blockIdx.x >> 3;
    const int tile = (rest / nrb) * 8 + xslot;
    if (tile >= ntiles) return;
    const int rb0 = (rest % nrb) * kLwRows;

    // a row block without a live row does nothing
    if (threadIdx.x == 0) s_any = 0;
    __syncthreads();
    for (int r = threadIdx.x; r < kLwRows; r += kLwThreads)
        if (rb0 + r < nrows && lm_row_live(rb0 + r, R, M_max, n_nodes, depth, status)) s_any = 1;
    __syncthreads();
    if (!s_any) return;

    const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(hidden), 0,
                                                                        static_cast<int>(h_bytes), kLmBufferFlags);
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(w), 0,
                                                                        static_cast<int>(w_bytes), kLmBufferFlags);
    // staging: thread t moves pieces q = t + 256 j of a block (row q / 16, piece q % 16);
    // rows past the tensor are clamped (computed, never merged)
    uint32_t soff[kLwStage];
#pragma unroll
    for (int j = 0; j < kLwStage; ++j) {
        int q = threadIdx.x + j * kLwThreads;
        q = q < kLwPiecesAll ? q : q - kLwPiecesAll;
        const int r = q / kLwPieces, pc = q % kLwPieces;
        int gr = rb0 + r;
        if (gr > nrows - 1) gr = nrows - 1;
        const int b = gr / R, u = gr - b * R;
        soff[j] = static_cast<uint32_t>((b * hsb + u * hsr) * 2 + pc * 16);
    }
    const int vbase = tile * kLwTile + wave * kLmVocabPerWave;
    uint32_t woff[2];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt) {
        int v = vbase + vt * 16 + c16;
        if (v > V - 1) v = V - 1;
        woff[vt] = static_cast<uint32_t>(v * wsr * 2 + G * 16);
    }
    lm_f32x4 acc[2][kLwRT];
#pragma unroll
    for (int vt = 0; vt < 2; ++vt)
#pragma unroll
        for (int rt = 0; rt < kLwRT; ++rt) acc[vt][rt] = lm_f32x4{0.f, 0.f, 0.f, 0.f};

    const int nblk = K / kLwKB, nsteps = K / 32;       // K a multiple of kLwBody kLwKB
    lm_u32x4 wa[kLwDepth][2];
    lm_u32x4 hv[kLwStage];
#pragma unroll
    for (int j = 0; j < kLwStage; ++j) hv[j] = __builtin_amdgcn_raw_buffer_load_b128(hr, soff[j], 0, 0);
    // the hidden states go out before the weights, as in the loop: then the loop's first
    // wait for them leaves the weights in flight
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kLwDepth; ++i)
#pragma unroll
        for (int vt = 0; vt < 2; ++vt) wa[i][vt] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[vt], i * 64, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
    for (int blk2 = 0; blk2 < nblk; blk2 += kLwBody) {
#pragma unroll
        for (int h = 0; h < kLwBody; ++h) {
            const int blk = blk2 + h;
            // stage block blk (after every wave is done with the last), then send for blk + 1
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kLwStage; ++j) {
                int q = threadIdx.x + j * kLwThreads;
                q = q < kLwPiecesAll ? q : q - kLwPiecesAll;
                const int r = q / kLwPieces, pc = q % kLwPieces;
                h_lds[r][pc ^ (r & 15)] = hv[j];
            }
            __syncthreads();
            // (the loads are unconditional -- the last block loads itself again -- so that the
            // compiler counts every load in flight exactly and never waits for the whole ring)
            const int nb = blk + 1 < nblk ? blk + 1 : nblk - 1;
#pragma unroll
            for (int j = 0; j < kLwStage; ++j)
                hv[j] = __builtin_amdgcn_raw_buffer_load_b128(hr, soff[j], nb * kLwKB * 2, 0);
#pragma unroll
            for (int ks = 0; ks < kLwSteps; ++ks) {
                const int slot = h * kLwSteps + ks;          // ring slot of step blk * 4 + ks
                // B operands read kLwPre row tiles ahead of their MFMAs (one wave's LDS reads
                // would otherwise wait one by one); the order is pinned below
                auto h_frag = [&](int rt) {
                    const int r = rt * 16 + c16;
                    return h_lds[r][(ks * 4 + G) ^ (r & 15)];
                };
                lm_u32x4 hq[kLwPre];
#pragma unroll
                for (int p = 0; p < kLwPre; ++p) hq[p] = h_frag(p);
#pragma unroll
                for (int rt = 0; rt < kLwRT; ++rt) {
                    const lm_u32x4 hb = hq[rt % kLwPre];
                    if (rt + kLwPre < kLwRT) hq[rt % kLwPre] = h_frag(rt + kLwPre);
#pragma unroll
                    for (int vt = 0; vt < 2; ++vt)
                        acc[vt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(lm_bf16x8, wa[slot][vt]), __builtin_bit_cast(lm_bf16x8, hb),
                            acc[vt][rt], 0, 0, 0);
                }
#pragma unroll
                for (int p = 0; p < kLwPre; ++p) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
#pragma unroll
                for (int rt = 0; rt < kLwRT; ++rt) {
                    if (rt + kLwPre < kLwRT) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                          // MFMA
                }
                int nxt = blk * kLwSteps + ks + kLwDepth;
                nxt = nxt < nsteps ? nxt : nsteps - 1;
#pragma unroll
                for (int vt = 0; vt < 2; ++vt)
                    wa[slot][vt] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[vt], nxt * 64, 0);
                // keep the loads where they are (the scheduler would sink them to their use)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // lane holds row rt*16 + c16 at entries vbase + vt*16 + G*4 + i
#pragma unroll
    for (int rt = 0; rt < kLwRT; ++rt) {
        uint64_t best = 0;
        bool nan = false;
#pragma unroll
        for (int vt = 0; vt < 2; ++vt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int v = vbase + vt * 16 + G * 4 + i;
                if (v < V) scan_one(acc[vt][rt][i], v, best, nan);
            }
        uint64_t k = nan ? kNanKey : best;
        uint64_t o = tmv::shfl_xor_u64(k, 16);
        k = o > k ? o : k;
        o = tmv::shfl_xor_u64(k, 32);
        k = o > k ? o : k;
        if (G == 0) s_key[wave][rt * 16 + c16] = k;
    }
    __syncthreads();
    for (int r = threadIdx.x; r < kLwRows; r += kLwThreads) {
        const int gr = rb0 + r;
        uint64_t k = s_key[0][r];
#pragma unroll
        for (int w2 = 1; w2 < kLwWaves; ++w2) k = s_key[w2][r] > k ? s_key[w2][r] : k;
        if (gr < nrows && lm_row_live(gr, R, M_max, n_nodes, depth, status))
            __hip_atomic_fetch_max(reinterpret_cast<unsigned long long *>(row_keys + gr),
                                   static_cast<unsigned long long>(k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// ============================================================== sampling
// K workgroups walk each sequence together, each owning a contiguous slice of the
// vocabulary.  At node u the teacher
// row p and the draft row q stay fixed while children are refused, and the residual left
// after j refusals is (p - c_j q)+ renormalised (c_{j+1} = c_j + sum (p - c_j q)+).  In
// integers the state is (M, T): R(y) = max(0, WP(y) SQ - WQ(y) M), T = sum R, and a
// refusal adds floor(T / SQ) to M.  So each thread quantises its entries of both rows
// once per node and keeps it in registers; a refusal is one pass of integer arithmetic
// over registers and one exact sum, and the test of any child needs only WP and WQ at its
// token.  The slices' partial sums meet at a per-sequence barrier of phase-tagged records
// in the workspace (bounded wait).
constexpr int kSampleThreads = 1024;
constexpr int kSampleWaves = kSampleThreads / kWave;
constexpr int kMaxNodes = 128;                 // tree nodes per sequence (host-checked)
constexpr int kMaxSlices = 64;                 // workgroups per sequence: one lane each at the barrier
constexpr int kMaxWords = 4 * ((kMaxNodes + 1 + 3) / 4);   // one per tried child, one draw
constexpr int kSeg = 16;                       // segment entries a thread keeps in registers
constexpr int kTailBatch = 4;                  // loads in flight per thread beyond them
constexpr uint64_t kTicksPerUs = 100;          // s_memrealtime runs at 100 MHz
constexpr uint32_t kDefaultWaitUs = 2000;       // tmv_tree_accept's wait bound
constexpr int kFlagBad = 1;                    // an entry outside [0, 1] in a scanned row
constexpr int kFlagTimeout = 2;                // a workgroup stopped waiting for the others
constexpr int kTagShift = 48;                  // record words: 48-bit piece | phase << 48
constexpr uint64_t kPieceMask = (1ull << kTagShift) - 1;
constexpr int kRowBufferFlags = 0x00020000;     // raw buffer descriptor word 3 (gfx9 family)

// a row as a buffer of `bytes` bytes: loads past the end return 0, so a segment's loads need
// neither a guard nor an address of their own (zero bytes: no load touches memory)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const float *row, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(row), 0, bytes, kRowBufferFlags);
}

__device__ __forceinline__ float row_load(__amdgpu_buffer_rsrc_t r, int x) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<uint32_t>(x) * 4u, 0, 0));
}

// Per-sequence synchronisation block of the workspace.  Record words carry the phase that
// wrote them, so a reader knows a record is current without a separate arrival count; a
// slot is rewritten two phases later only after every slice has read it.  Between calls
// everything is zero: the last workgroup to leave clears the records and the count.
struct SeqSync {
    uint64_t leave;                          // workgroups done with this call
    uint64_t failed;                         // set by a workgroup that stopped waiting
    uint64_t pad[14];
    uint64_t rec[2][kMaxSlices][4];          // [phase parity][slice]: sum bits 0-47, 48-95, 96-143; flags
};

struct SeqView {
    u128 own;        // this slice's partial sum
    u128 total;      // sum over the slices
    u128 before;     // sum over the slices before this one
    int flags;       // OR of the slices' flags, plus kFlagTimeout if this workgroup gave up
};

struct SyncLds {
    u128 red[kSampleThreads];   // every thread's term of the block sum
    int fl[kSampleWaves];       // per wave: any flag raised
    u128 res[3];         // total, before, own
    int res_flags;
    uint64_t dec_m;      // decision for the next child (taken by wave 0): M after a refusal,
    int dec_accept;      // and whether the child is accepted
};

// wave-uniform copies in scalar registers (the values are equal in every lane)
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ u128 uniform_u128(u128 v) {
    return (static_cast<u128>(uniform_u64(static_cast<uint64_t>(v >> 64))) << 64) | uniform_u64(static_cast<uint64_t>(v));
}

// floor(p * 2^31) for p in [0, 1] (at most 2^31); flags entries outside [0, 1] and NaN
__device__ __forceinline__ uint32_t quantise31(float p, int &bad) {
    // p = m * 2^(e - 150) with m the 24-bit significand, so p * 2^31 = m * 2^(e - 119):
    // an exact integer operation on the fp32 bits
    const uint32_t u = __float_as_uint(p);
    if (u > 0x3F800000u) {                     // above 1, negative, infinite or NaN
        if (u != 0x80000000u) bad = 1;         // (-0 is zero)
        return 0;
    }
    const uint32_t e = u >> 23;
    const uint32_t m = (u & 0x7FFFFFu) | 0x800000u;
    if (e >= 119) return m << (e - 119);       // e <= 127: at most 2^31
    const uint32_t sh = 119 - e;
    return sh >= 24 ? 0u : m >> sh;            // zero and subnormals give 0
}

// R(y) = max(0, WP(y) SQ - WQ(y) M) < 2^96 from four 32 x 32 -> 64-bit products, as its low
// 32 bits and the rest: R = lo + hi * 2^32
struct R96 {
    uint32_t lo;
    uint64_t hi;
};

// kWideSQ / kWideM: whether SQ / M may exceed 32 bits (when not, their high products vanish;
// normalised rows give SQ < 2^32, and M < 2^32 until c_j reaches about 2)
template <bool kWideSQ = true, bool kWideM = true>
__device__ __forceinline__ R96 resid96(uint32_t wp, uint32_t wq, uint64_t SQ, uint64_t M) {
    const uint64_t a_lo = static_cast<uint64_t>(wp) * static_cast<uint32_t>(SQ);
    const uint64_t a_hi = kWideSQ ? static_cast<uint64_t>(wp) * static_cast<uint32_t>(SQ >> 32) : 0;
    const uint64_t c_lo = static_cast<uint64_t>(wq) * static_cast<uint32_t>(M);
    const uint64_t c_hi = kWideM ? static_cast<uint64_t>(wq) * static_cast<uint32_t>(M >> 32) : 0;
    const uint64_t a12 = (a_lo >> 32) + a_hi, c12 = (c_lo >> 32) + c_hi;   // (neither sum wraps)
    const uint32_t a0 = static_cast<uint32_t>(a_lo), c0 = static_cast<uint32_t>(c_lo);
    // a - c as lo + d12 * 2^32 with a signed high part (a12 < 2^55, c12 < 2^63: no overflow);
    // it is negative exactly when a < c, and its sign masks both parts
    const int64_t d12 = static_cast<int64_t>(a12 - c12 - (a0 < c0 ? 1u : 0u));
    const uint64_t keep = ~static_cast<uint64_t>(d12 >> 63);
    R96 r;
    r.lo = (a0 - c0) & static_cast<uint32_t>(keep);
    r.hi = static_cast<uint64_t>(d12) & keep;
    return r;
}

__device__ __forceinline__ u128 resid(uint32_t wp, uint32_t wq, uint64_t SQ, uint64_t M) {
    const R96 r = resid96(wp, wq, SQ, M);
    return (static_cast<u128>(r.hi) << 32) | r.lo;
}

// a * b as three 64-bit words, least significant first
__device__ __forceinline__ void mul_u128_u64(u128 a, uint64_t b, uint64_t w[3]) {
    const u128 lo = static_cast<u128>(static_cast<uint64_t>(a)) * b;
    const u128 hi = static_cast<u128>(static_cast<uint64_t>(a >> 64)) * b;
    const u128 mid = (lo >> 64) + static_cast<uint64_t>(hi);
    w[0] = static_cast<uint64_t>(lo);
    w[1] = static_cast<uint64_t>(mid);
    w[2] = static_cast<uint64_t>(hi >> 64) + static_cast<uint64_t>(mid >> 64);
}

// accept iff U * WQ(x) * T < R(x) * SQ * 2^24 (both sides below 2^166)
__device__ __forceinline__ bool sample_accepts(uint64_t U, uint32_t wqx, u128 T, u128 rx, uint64_t SQ) {
    uint64_t l[3], r[3];
    mul_u128_u64(T, U * wqx, l);
    mul_u128_u64(rx << 24, SQ, r);
    if (l[2] != r[2]) return l[2] < r[2];
    if (l[1] != r[1]) return l[1] < r[1];
    return l[0] < r[0];
}

// floor(n / d) for d >= 1 and a quotient below 2^64: a double-precision estimate, then
// exact corrections (the estimate is off by a few units at most)
__device__ uint64_t udiv_u128_u64(u128 n, uint64_t d) {
    const double est = (static_cast<double>(static_cast<uint64_t>(n >> 64)) * 18446744073709551616.0 +
                        static_cast<double>(static_cast<uint64_t>(n))) / static_cast<double>(d);
    uint64_t q = est >= 18446744073709549568.0 ? 0xFFFFFFFFFFFFF800ull : static_cast<uint64_t>(est);
    u128 prod = static_cast<u128>(q) * d;
    while (prod > n) { --q; prod -= d; }
    while (n - prod >= d) { ++q; prod += d; }
    return q;
}

// floor((word >> 32) * T / 2^32), split so that no product exceeds 128 bits
__device__ __forceinline__ u128 draw_target(uint64_t word, u128 T) {
    const uint64_t h = word >> 32;
    return static_cast<u128>(h) * (T >> 32) + ((static_cast<u128>(h) * static_cast<uint32_t>(T)) >> 32);
}

// true in every thread if v is true in any thread of the block
__device__ bool block_any(bool v, int *sh) {
    __syncthreads();
    if (threadIdx.x == 0) *sh = 0;
    __syncthreads();
    if (__ballot(v) != 0 && (threadIdx.x & (kWave - 1)) == 0) *sh = 1;
    __syncthreads();
    return *sh != 0;
}

// Sum `local` over the block and then over the K slices of the sequence.  Every thread
// of the block calls it; `phase` counts the calls and advances alike in all K.  Wave 0,
// which gathers the slices' sums, then runs post(view) -- the walk's scalar decisions are
// taken there once, instead of in every wave -- before the block reads the results.
template <class Post>
__device__ SeqView seq_reduce(SeqSync *ss, int K, int k, int &phase, u128 local, int flags, SyncLds &L,
                             uint64_t wait_ticks, Post post) {
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const bool any_bad = __ballot(flags != 0) != 0;
    __syncthreads();                                  // the previous call's results are read
    L.red[threadIdx.x] = local;
    if (lane == 0) L.fl[wv] = any_bad ? 1 : 0;
    __syncthreads();
    const uint64_t tag = static_cast<uint64_t>(++phase);
    if (wv == 0) {
        // the block's sum: each lane adds sixteen staged terms, then one wave reduction
        u128 part = 0;
#pragma unroll
        for (int j = 0; j < kSampleThreads / kWave; ++j) part += L.red[j * kWave + lane];
        const u128 wg = tmv::wave_sum_u128(part);
        const int fl = __ballot(lane < kSampleWaves && L.fl[lane] != 0) != 0 ? kFlagBad : 0;
        const uint64_t own[4] = {static_cast<uint64_t>(wg) & kPieceMask, static_cast<uint64_t>(wg >> 48) & kPieceMask,
                                 static_cast<uint64_t>(wg >> 96) & kPieceMask, static_cast<uint64_t>(fl)};
        uint64_t *slot = &ss->rec[tag & 1][0][0];
        if (lane < 4) {
            const uint64_t word = (lane == 0 ? own[0] : lane == 1 ? own[1] : lane == 2 ? own[2] : own[3]) | (tag << kTagShift);
            __hip_atomic_store(slot + 4 * k + lane, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // lane j < K collects slice j's record (its own from registers)
        uint64_t w0 = own[0], w1 = own[1], w2 = own[2], w3 = own[3];
        bool ok = lane >= K || lane == k;
        int timed_out = 0;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        for (;;) {
            if (!ok) {
                const uint64_t *r = slot + 4 * lane;
                w0 = __hip_atomic_load(r + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                w1 = __hip_atomic_load(r + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                w2 = __hip_atomic_load(r + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                w3 = __hip_atomic_load(r + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                ok = (w0 >> kTagShift) == tag && (w1 >> kTagShift) == tag && (w2 >> kTagShift) == tag &&
                     (w3 >> kTagShift) == tag;
            }
            if (__ballot(!ok) == 0) break;
            if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks) { timed_out = 1; break; }
            __builtin_amdgcn_s_sleep(1);
        }
        // the slices' sums in scalar registers, slice by slice (K is at most 64)
        const bool rec_bad = __ballot(lane < K && (w3 & kPieceMask) != 0) != 0;
        u128 tot = 0, bef = 0;
        for (int j = 0; j < K; ++j) {
            const uint32_t a0 = __builtin_amdgcn_readlane(static_cast<uint32_t>(w0), j);
            const uint32_t a1 = __builtin_amdgcn_readlane(static_cast<uint32_t>(w0 >> 32), j);
            const uint32_t b0 = __builtin_amdgcn_readlane(static_cast<uint32_t>(w1), j);
            const uint32_t b1 = __builtin_amdgcn_readlane(static_cast<uint32_t>(w1 >> 32), j);
            const uint32_t c0 = __builtin_amdgcn_readlane(static_cast<uint32_t>(w2), j);
            const uint32_t c1 = __builtin_amdgcn_readlane(static_cast<uint32_t>(w2 >> 32), j);
            const u128 vj = (static_cast<u128>(((static_cast<uint64_t>(c1) << 32) | c0) & kPieceMask) << 96) |
                            (static_cast<u128>(((static_cast<uint64_t>(b1) << 32) | b0) & kPieceMask) << 48) |
                            (((static_cast<uint64_t>(a1) << 32) | a0) & kPieceMask);
            if (j < k) bef += vj;
            tot += vj;
        }
        const int fj = (rec_bad ? kFlagBad : 0) | (timed_out ? kFlagTimeout : 0);
        if (lane == 0) {
            L.res[0] = tot;
            L.res[1] = bef;
            L.res[2] = wg;
            L.res_flags = fj;
        }
        SeqView w;
        w.total = tot;
        w.before = bef;
        w.own = uniform_u128(wg);
        w.flags = fj;
        post(w);
    }
    __syncthreads();
    SeqView r;
    r.total = uniform_u128(L.res[0]);
    r.before = uniform_u128(L.res[1]);
    r.own = uniform_u128(L.res[2]);
    r.flags = __builtin_amdgcn_readfirstlane(L.res_flags);
    return r;
}

// The workgroup is done with the call.  Its record and output stores (all written through
// to memory) are complete before it counts itself out, so the last of the K sees every
// other workgroup's effects: it clears every record for the next call, and when any
// workgroup gave up waiting it writes the sequence's failed state last -- status
// TMV_ERR_DEVICE and zero outputs, whatever a slice that did finish the walk wrote.
__device__ __forceinline__ void store_out(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ void seq_leave(SeqSync *ss, int K, int b, int D_max, int32_t *__restrict__ status,
                          int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                          int32_t *__restrict__ next_token) {
    __builtin_amdgcn_s_waitcnt(0);                    // every wave's stores are complete
    __syncthreads();
    if (threadIdx.x < kWave) {
        const int lane = threadIdx.x;
        uint64_t l = 0;
        if (lane == 0) {
            __builtin_amdgcn_s_waitcnt(0);
            l = __hip_atomic_fetch_add(&ss->leave, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        l = __shfl(l, 0, kWave);
        if (l == static_cast<uint64_t>(K) - 1) {
            const bool failed = __hip_atomic_load(&ss->failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
            if (failed) {
                for (int j = lane; j < D_max; j += kWave) store_out(path + static_cast<int64_t>(b) * D_max + j, 0);
                if (lane == 0) {
                    store_out(accept_len + b, 0);
                    store_out(next_token + b, 0);
                    store_out(status + b, TMV_ERR_DEVICE);
                    __hip_atomic_store(&ss->failed, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            for (int i = lane; i < 2 * K * 4; i += kWave) {
                const int slot = i / (4 * K), j = i % (4 * K);
                __hip_atomic_store(&ss->rec[slot][j / 4][j % 4], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            if (lane == 0) __hip_atomic_store(&ss->leave, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Slice layout: column c of a slice is the 1024 entries x_lo + c * kSampleThreads + [0,
// kSampleThreads), so thread t holds entry t of every column and each column is read with
// fully coalesced loads.  Columns 0 .. kSeg-1 live in registers; later ones (only when a
// slice exceeds kSampleThreads * kSeg entries) are read and quantised again when needed.

// f(c, WP, WQ) for this thread's entry of every column c >= kSeg (WP = WQ = 0 past the slice)
template <class F>
__device__ __forceinline__ void visit_tail_columns(int x_lo, int x_hi, int ncol, __amdgpu_buffer_rsrc_t prs,
                                                   __amdgpu_buffer_rsrc_t qrs, F f) {
    for (int c0 = kSeg; c0 < ncol; c0 += kTailBatch) {
        float tp[kTailBatch], tq[kTailBatch];
#pragma unroll
        for (int e = 0; e < kTailBatch; ++e) {
            const int x = x_lo + (c0 + e) * kSampleThreads + static_cast<int>(threadIdx.x);
            tp[e] = row_load(prs, x);
            tq[e] = row_load(qrs, x);
        }
        int unused = 0;
#pragma unroll
        for (int e = 0; e < kTailBatch; ++e) {
            const bool in = c0 + e < ncol && x_lo + (c0 + e) * kSampleThreads + static_cast<int>(threadIdx.x) < x_hi;
            f(c0 + e, quantise31(in ? tp[e] : 0.f, unused), quantise31(in ? tq[e] : 0.f, unused));
        }
    }
}

// this thread's sum of R over the register columns, in two 64-bit halves (each below 2^59)
template <bool kWideSQ, bool kWideM>
__device__ __forceinline__ void register_sum(const uint32_t (&rp)[kSeg], const uint32_t (&rq)[kSeg], uint64_t SQ,
                                             uint64_t M, uint64_t &lo, uint64_t &hi) {
#pragma unroll
    for (int e = 0; e < kSeg; ++e) {
        // (opaque copies: the compiler would otherwise keep 64-bit widened copies of the
        // cached rows alive across the refusal loop)
        uint32_t wp = rp[e], wq = rq[e];
        asm volatile("" : "+v"(wp), "+v"(wq));
        const R96 r = resid96<kWideSQ, kWideM>(wp, wq, SQ, M);
        lo += r.lo;
        hi += r.hi;
    }
}

// this thread's sum of R over its entries of the slice
__device__ __forceinline__ u128 thread_sum(const uint32_t (&rp)[kSeg], const uint32_t (&rq)[kSeg], int x_lo,
                                           int x_hi, int ncol, __amdgpu_buffer_rsrc_t prs,
                                           __amdgpu_buffer_rsrc_t qrs, uint64_t SQ, uint64_t M) {
    uint64_t lo = 0, hi = 0;
    const bool wide_sq = (SQ >> 32) != 0, wide_m = (M >> 32) != 0;      // (wave-uniform)
    if (wide_sq) {
        if (wide_m) register_sum<true, true>(rp, rq, SQ, M, lo, hi);
        else register_sum<true, false>(rp, rq, SQ, M, lo, hi);
    } else {
        if (wide_m) register_sum<false, true>(rp, rq, SQ, M, lo, hi);
        else register_sum<false, false>(rp, rq, SQ, M, lo, hi);
    }
    u128 s = static_cast<u128>(lo) + (static_cast<u128>(hi) << 32);
    visit_tail_columns(x_lo, x_hi, ncol, prs, qrs, [&](int, uint32_t a, uint32_t c2) { s += resid(a, c2, SQ, M); });
    return s;
}

__global__ void __launch_bounds__(kSampleThreads)
sample_walk_kernel(int M_max, int D_max, int V, int K,
                   const int32_t *__restrict__ tokens,
                   const float *__restrict__ p, int64_t psb, int64_t psr,
                   const float *__restrict__ q, int64_t qsb, int64_t qsr,
                   uint64_t seed, uint64_t step,
                   const int32_t *__restrict__ n_nodes, const int32_t *__restrict__ anc,
                   const int32_t *__restrict__ depth, int32_t *__restrict__ status,
                   int32_t *__restrict__ accept_len, int32_t *__restrict__ path,
                   int32_t *__restrict__ next_token, SeqSync *__restrict__ sync, uint64_t wait_ticks)
{
    __shared__ SyncLds L;
    __shared__ int par[kMaxNodes + 1];         // parent of a live node, -1 otherwise
    __shared__ int tok[kMaxNodes + 1];         // draft token of a live node
    __shared__ int kids[kMaxNodes];
    __shared__ int kid_count[kSampleWaves];
    __shared__ int nkids;
    __shared__ uint32_t kwp[kMaxNodes], kwq[kMaxNodes];   // WP and WQ at the children's tokens
    __shared__ uint32_t rows_lds[2][kSeg * kSampleThreads]; // draw: one chunk of the slice, in x order
    __shared__ u128 scan_sh[kSampleWaves];
    __shared__ int flag_sh;
    __shared__ int draw_tok;
    __shared__ uint64_t words[kMaxWords];                 // the walk's random words, in order

    const int b = blockIdx.x / K, k = blockIdx.x % K, tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    const int x_lo = static_cast<int>(static_cast<int64_t>(V) * k / K);
    const int x_hi = static_cast<int>(static_cast<int64_t>(V) * (k + 1) / K);
    const int ncol = (x_hi - x_lo + kSampleThreads - 1) / kSampleThreads;
    SeqSync *ss = sync + b;
    int phase = 0;
    const int R = M_max + 1, W = D_max + 1;
    const int M = n_nodes[b];
    int32_t *pth = path + static_cast<int64_t>(b) * D_max;
    const int st_in = status[b];
    const int st = (st_in == TMV_OK && (M < 0 || M > M_max)) ? TMV_ERR_INPUT : st_in;
    const uint64_t stream = (step << 32) | static_cast<uint32_t>(b);

    // outputs: slice 0 writes the path, the length and a data error; the slice holding the
    // final draw writes the token.  A workgroup that gave up waiting (TMV_ERR_DEVICE) only
    // marks the sequence failed; the last workgroup to leave writes the failed state.  All
    // output stores are written through, so that the last one to leave writes last.
    auto finish = [&](int code, int acc, int tk, bool mine) {
        __syncthreads();
        if (code == TMV_ERR_DEVICE) {
            if (tid == 0) __hip_atomic_store(&ss->failed, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (code != TMV_OK) { acc = 0; tk = 0; }
            if (k == 0)
                for (int j = tid; j < D_max; j += kSampleThreads)
                    if (code != TMV_OK || j >= acc) store_out(pth + j, 0);
            if (tid == 0) {
                if (k == 0) {
                    store_out(accept_len + b, acc);
                    if (code != TMV_OK) {
                        store_out(next_token + b, 0);
                        if (st_in == TMV_OK) store_out(status + b, code);
                    }
                }
                if (code == TMV_OK && mine) store_out(next_token + b, tk);
            }
        }
        seq_leave(ss, K, b, D_max, status, accept_len, path, next_token);
    };
    if (st != TMV_OK) { finish(st, 0, 0, false); return; }

    const float *p_b = p + b * psb, *q_b = q + b * qsb;

    // the random words the walk can consume (one per tried child and one draw), computed
    // once: Philox blocks at counters 1, 2, ... hold words 0-3, 4-7, ...
    if (tid < kMaxWords / 4) {
        uint64_t o[4];
        tmv::philox4x64_10(static_cast<uint64_t>(tid) + 1, seed, stream, o);
#pragma unroll
        for (int j = 0; j < 4; ++j) words[4 * tid + j] = o[j];
    }
    // the live nodes' parents and tokens (every slice checks every token: one answer)
    bool bad_tok = false;
    for (int c = tid; c <= M_max; c += kSampleThreads) {
        int pc = -1, t = 0;
        if (c >= 1 && c <= M && W > 1 && depth[static_cast<int64_t>(b) * R + c] >= 1) {
            pc = anc[(static_cast<int64_t>(b) * R + c) * W + 1];
            t = tokens[static_cast<int64_t>(b) * R + c];
            if (t < 0 || t >= V) bad_tok = true;
        }
        par[c] = pc;
        tok[c] = t;
    }
    if (block_any(bad_tok, &flag_sh)) { finish(TMV_ERR_INPUT, 0, 0, false); return; }

    uint32_t rp[kSeg], rq[kSeg];
    uint64_t n = 0;            // random words consumed
    int u = 0, acc = 0;
    for (;;) {
        // children of u in ascending id: thread c-1 tests node c, compacted with ballots
        {
            const int c = tid + 1;
            const bool is_kid = c <= M_max && par[c] == u;
            const uint64_t bal = __ballot(is_kid);
            if (lane == 0) kid_count[wv] = __popcll(bal);
            __syncthreads();
            if (is_kid) {
                int before = __popcll(bal & ((1ull << lane) - 1));
                for (int w2 = 0; w2 < wv; ++w2) before += kid_count[w2];
                kids[before] = c;
            }
            if (tid == 0) {
                int kk = 0;
                for (int w2 = 0; w2 < kSampleWaves; ++w2) kk += kid_count[w2];
                nkids = kk;
            }
            __syncthreads();
        }
        const int nk = nkids;
        const bool have_q = nk > 0;          // a leaf's q row is never read
        const __amdgpu_buffer_rsrc_t prs = row_buffer(p_b + static_cast<int64_t>(u) * psr, V * 4);
        const __amdgpu_buffer_rsrc_t qrs = row_buffer(q_b + static_cast<int64_t>(u) * qsr, have_q ? V * 4 : 0);

        // arrival at u: quantise this thread's entries of both rows into registers, sum
        // them, and fetch both rows at the children's tokens
        int bd = 0;
        uint64_t sp = 0, sq = 0;
        {
            float fp[kSeg], fq[kSeg];
#pragma unroll
            for (int e = 0; e < kSeg; ++e) {
                const int x = x_lo + e * kSampleThreads + tid;
                fp[e] = row_load(prs, x);
                fq[e] = row_load(qrs, x);
            }
            const int xc = tid < nk ? tok[kids[tid]] : 0;
            const float cp = row_load(prs, xc), cq = row_load(qrs, xc);
#pragma unroll
            for (int e = 0; e < kSeg; ++e) {
                const bool in = x_lo + e * kSampleThreads + tid < x_hi;
                rp[e] = quantise31(in ? fp[e] : 0.f, bd);
                rq[e] = quantise31(in ? fq[e] : 0.f, bd);
                sp += rp[e];
                sq += rq[e];
            }
            for (int c0 = kSeg; c0 < ncol; c0 += kTailBatch) {
                float tp[kTailBatch], tq[kTailBatch];
#pragma unroll
                for (int e = 0; e < kTailBatch; ++e) {
                    const int x = x_lo + (c0 + e) * kSampleThreads + tid;
                    tp[e] = row_load(prs, x);
                    tq[e] = row_load(qrs, x);
                }
#pragma unroll
                for (int e = 0; e < kTailBatch; ++e)
                    if (c0 + e < ncol && x_lo + (c0 + e) * kSampleThreads + tid < x_hi) {
                        sp += quantise31(tp[e], bd);
                        sq += quantise31(tq[e], bd);
                    }
            }
            if (tid < nk) {
                int unused = 0;
                kwp[tid] = quantise31(cp, unused);
                kwq[tid] = quantise31(cq, unused);
            }
        }
        // The decision on child ci against state (M, T): its random word, the accept test,
        // and after a refusal the next threshold M + floor(T / SQ).  Taken by wave 0.
        auto decide = [&](int ci, uint64_t Md, u128 Td, uint64_t SQd) {
            int accept = 0;
            uint64_t m_next = 0;
            if (ci < nk) {
                const uint64_t U = words[n + ci] >> 40;
                const uint32_t wpx = __builtin_amdgcn_readfirstlane(kwp[ci]);
                const uint32_t wqx = __builtin_amdgcn_readfirstlane(kwq[ci]);
                accept = sample_accepts(U, wqx, Td, resid(wpx, wqx, SQd, Md), SQd) ? 1 : 0;
                if (!accept) m_next = Md + udiv_u128_u64(Td, SQd);
            }
            if (lane == 0) {
                L.dec_accept = accept;
                L.dec_m = m_next;
            }
        };
        // (slice sums of WP and WQ stay below 2^55, so they share one 128-bit sum)
        const SeqView va = seq_reduce(ss, K, k, phase, static_cast<u128>(sp) | (static_cast<u128>(sq) << 64),
                                      bd ? kFlagBad : 0, L, wait_ticks, [&](const SeqView &w) {
            const uint64_t sp_w = static_cast<uint64_t>(w.total), sq_w = static_cast<uint64_t>(w.total >> 64);
            if (!(w.flags & (kFlagBad | kFlagTimeout)) && sp_w != 0 && (!have_q || sq_w != 0)) {
                const uint64_t sq1 = have_q ? sq_w : 1;
                decide(0, 0, static_cast<u128>(sp_w) * sq1, sq1);
            }
        });
        if (va.flags & kFlagTimeout) { finish(TMV_ERR_DEVICE, 0, 0, false); return; }
        const uint64_t SP = static_cast<uint64_t>(va.total), SQt = static_cast<uint64_t>(va.total >> 64);
        if ((va.flags & kFlagBad) || SP == 0 || (have_q && SQt == 0)) { finish(TMV_ERR_INPUT, 0, 0, false); return; }
        const uint64_t SQ = have_q ? SQt : 1;

        // state on arrival: M = 0, R = WP * SQ
        uint64_t Mc = 0;
        u128 T = static_cast<u128>(SP) * SQ;
        u128 own = static_cast<u128>(static_cast<uint64_t>(va.own)) * SQ;    // this slice's share
        u128 before = static_cast<u128>(static_cast<uint64_t>(va.before)) * SQ;
        bool moved = false;
        for (int ci = 0; ci < nk; ++ci) {
            if (__builtin_amdgcn_readfirstlane(L.dec_accept)) {
                if (k == 0 && tid == 0) store_out(pth + acc, kids[ci]);
                ++acc;
                u = kids[ci];
                n += ci + 1;
                moved = true;
                break;
            }
            // refusal: the residual against q is the state at M + T / SQ
            const uint64_t Mn = uniform_u64(L.dec_m);
            // (SQ is made opaque here so that the products WP * SQ are not hoisted out of
            // the refusal loop: sixteen of them would not fit next to the cached rows)
            uint64_t SQp = SQ;
            asm volatile("" : "+s"(SQp));
            const u128 s = thread_sum(rp, rq, x_lo, x_hi, ncol, prs, qrs, SQp, Mn);
            const SeqView vr = seq_reduce(ss, K, k, phase, s, 0, L, wait_ticks, [&](const SeqView &w) {
                if (!(w.flags & kFlagTimeout)) {
                    if (w.total != 0) decide(ci + 1, Mn, w.total, SQ);
                    else decide(ci + 1, Mc, T, SQ);      // empty residual: the state is kept
                }
            });
            if (vr.flags & kFlagTimeout) { finish(TMV_ERR_DEVICE, 0, 0, false); return; }
            if (vr.total != 0) {               // an empty residual keeps the state
                Mc = Mn;
                T = vr.total;
                own = vr.own;
                before = vr.before;
            }
        }
        if (moved) continue;
        n += nk;

        // Draw the bonus (no children) or the correction (all refused): the token is the
        // first x whose running sum of R exceeds t.  The slice sums locate the slice.
        // Inside it, groups of kSeg columns are summed column by column until the group
        // holding t is found; an exclusive scan over the threads of that column ends it.
        const u128 t = draw_target(words[n], T);
        const bool mine = before <= t && t < before + own;
        int tk = 0;
        if (mine) {
            // The slice in chunks of kSeg columns (kSeg * kSampleThreads entries), each staged
            // in LDS in x order -- the first from the registers, which makes them free for
            // the draw -- so that thread i holds entries [kSeg i, kSeg i + kSeg) of the chunk.
            u128 base = before;             // running sum before the current chunk
            int found = -1;
#pragma unroll
            for (int e = 0; e < kSeg; ++e) {
                rows_lds[0][e * kSampleThreads + tid] = rp[e];
                rows_lds[1][e * kSampleThreads + tid] = rq[e];
            }
            for (int c0 = 0; c0 < ncol && found < 0; c0 += kSeg) {
                if (c0 > 0) {
                    __syncthreads();                      // (the previous chunk is read)
#pragma unroll
                    for (int e = 0; e < kSeg; ++e) {
                        const int x = x_lo + (c0 + e) * kSampleThreads + tid;
                        const bool in = c0 + e < ncol && x < x_hi;
                        const float fpv = row_load(prs, x), fqv = row_load(qrs, x);
                        int unused = 0;
                        rows_lds[0][e * kSampleThreads + tid] = in ? quantise31(fpv, unused) : 0u;
                        rows_lds[1][e * kSampleThreads + tid] = in ? quantise31(fqv, unused) : 0u;
                    }
                }
                __syncthreads();
                u128 mine_sum = 0;
#pragma unroll
                for (int i = 0; i < kSeg; ++i)
                    mine_sum += resid(rows_lds[0][kSeg * tid + i], rows_lds[1][kSeg * tid + i], SQ, Mc);
                // exclusive scan of the threads' sums (the chunk total comes with it)
                u128 incl = mine_sum;
                for (int o = 1; o < kWave; o <<= 1) {
                    u128 y = 0;
#pragma unroll
                    for (int part = 0; part < 4; ++part) {
                        const uint32_t v32 = static_cast<uint32_t>(incl >> (32 * part));
                        y |= static_cast<u128>(static_cast<uint32_t>(__shfl_up(static_cast<int>(v32), o, kWave))) << (32 * part);
                    }
                    if (lane >= o) incl += y;
                }
                if (lane == kWave - 1) scan_sh[wv] = incl;
                if (tid == 0) draw_tok = -1;
                __syncthreads();
                u128 excl = base + incl - mine_sum, chunk = 0;
                for (int w2 = 0; w2 < kSampleWaves; ++w2) {
                    if (w2 < wv) excl += scan_sh[w2];
                    chunk += scan_sh[w2];
                }
                if (mine_sum > 0 && excl <= t && t < excl + mine_sum) {
                    u128 cum = excl;
                    int f = -1;
                    for (int i = 0; i < kSeg && f < 0; ++i) {
                        cum += resid(rows_lds[0][kSeg * tid + i], rows_lds[1][kSeg * tid + i], SQ, Mc);
                        if (cum > t) f = i;
                    }
                    draw_tok = x_lo + c0 * kSampleThreads + kSeg * tid + (f < 0 ? kSeg - 1 : f);
                }
                __syncthreads();
                found = __builtin_amdgcn_readfirstlane(draw_tok);
                base = uniform_u128(base + chunk);
            }
            tk = found >= 0 ? found : x_hi - 1;   // (found is always set: t lies in this slice)
        }
        finish(TMV_OK, acc, tk, mine);
        return;
    }
}

}  // namespace

// greedy workspace, one-launch part: keys and counters (all zero between calls)
static size_t greedy_fused_bytes(int B, int M_max) {
    return (2 * static_cast<size_t>(B) * (M_max + 1) + B) * kSlot;
}

// workgroups of the one-launch greedy kernel resident at once on an otherwise idle device
// (its occupancy per compute unit times the compute units); larger scans take two launches
static int64_t greedy_resident() {
    static std::mutex mu;
    static int64_t cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void *>(&greedy_accept_kernel<TMV_F32>), kScanThreads, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        cached[dev] = static_cast<int64_t>(cus) * per_cu;
    }
    return cached[dev];
}

// sampling workspace: one synchronisation block per sequence (all zero between calls)
static size_t sample_ws_bytes(int B) {
    return static_cast<size_t>(B) * sizeof(SeqSync) + 256;
}

// workgroups per sequence: all B * K of the launch resident at once on an otherwise idle
// device (the walk kernel's occupancy per compute unit times the compute units), at most
// kMaxSlices, slices of >= 2048 entries.  The walk's results do not depend on K.
static int walk_capacity() {
    static std::mutex mu;
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(&sample_walk_kernel),
                                                         kSampleThreads, 0) != hipSuccess || per_cu < 1)
            per_cu = 1;
        cached[dev] = cus * per_cu;
    }
    return cached[dev];
}

static int sample_slices(int B, int V) {
    int K = walk_capacity() / (B > 0 ? B : 1);
    if (K > kMaxSlices) K = kMaxSlices;
    if (K > V / 2048) K = V / 2048;
    return K < 1 ? 1 : K;
}

extern "C" size_t tmv_tree_accept_workspace(int mode, int B, int M_max, int V)
{
    if (B <= 0 || M_max < 0 || V <= 0) return 256;
    if (mode == TMV_ACCEPT_GREEDY) {
        const int nchunk = (V + kScanChunk - 1) / kScanChunk;
        return greedy_fused_bytes(B, M_max) + static_cast<size_t>(B) * (M_max + 1) * nchunk * sizeof(uint64_t) + 256;
    }
    return sample_ws_bytes(B);
}

extern "C" int tmv_tree_accept_wait(int mode, int B, int M_max, int D_max, int V,
                                    const int32_t *tokens, int row_dtype, const void *teacher,
                                    int64_t t_stride_b, int64_t t_stride_row,
                                    const float *draft_q, int64_t q_stride_b, int64_t q_stride_row,
                                    uint64_t seed, uint64_t step,
                                    const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                                    int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token,
                                    void *workspace, size_t workspace_bytes, uint32_t wait_us, void *stream)
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
        if (blocks <= greedy_resident()) {
            if (row_dtype == TMV_F32)
                hipLaunchKernelGGL(greedy_accept_kernel<TMV_F32>, dim3(static_cast<unsigned>(blocks)), dim3(kScanThreads),
                                   0, s, M_max, D_max, V, nchunk, teacher, t_stride_b, t_stride_row, tokens, n_nodes, anc,
                                   depth, status, accept_len, path, next_token, ws);
            else
                hipLaunchKernelGGL(greedy_accept_kernel<TMV_BF16>, dim3(static_cast<unsigned>(blocks)), dim3(kScanThreads),
                                   0, s, M_max, D_max, V, nchunk, teacher, t_stride_b, t_stride_row, tokens, n_nodes, anc,
                                   depth, status, accept_len, path, next_token, ws);
            return tmv_host::launch_status(hipGetLastError());
        }
        uint64_t *keys = reinterpret_cast<uint64_t *>(ws + greedy_fused_bytes(B, M_max));
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
    if (V > (1 << 24)) return TMV_ERR_ARG;
    const int K = sample_slices(B, V);
    hipLaunchKernelGGL(sample_walk_kernel, dim3(static_cast<unsigned>(B) * K), dim3(kSampleThreads), 0, s, M_max,
                       D_max, V, K, tokens, static_cast<const float *>(teacher), t_stride_b, t_stride_row, draft_q,
                       q_stride_b, q_stride_row, seed, step, n_nodes, anc, depth, status, accept_len, path,
                       next_token, reinterpret_cast<SeqSync *>(ws), static_cast<uint64_t>(wait_us) * kTicksPerUs);
    return tmv_host::launch_status(hipGetLastError());
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
    return tmv_tree_accept_wait(mode, B, M_max, D_max, V, tokens, row_dtype, teacher, t_stride_b, t_stride_row, draft_q,
                                q_stride_b, q_stride_row, seed, step, n_nodes, anc, depth, status, accept_len, path,
                                next_token, workspace, workspace_bytes, kDefaultWaitUs, stream);
}

extern "C" size_t tmv_tree_accept_lm_head_workspace(int B, int M_max)
{
    if (B <= 0 || M_max < 0) return 256;
    return static_cast<size_t>(B) * (M_max + 1) * sizeof(uint64_t) + 256;
}

extern "C" int tmv_tree_accept_lm_head(int B, int M_max, int D_max, int K, int V, const int32_t *tokens,
                                       const void *hidden, int64_t h_stride_b, int64_t h_stride_row,
                                       const void *lm_head, int64_t w_stride_row,
                                       const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                                       int32_t *status, int32_t *accept_len, int32_t *path, int32_t *next_token,
                                       int32_t *row_argmax, void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 0 || M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128 || V < 1) return TMV_ERR_ARG;
    if ((K != 512 && K != 1024 && K != 2048 && K != 4096 && K != 8192) || h_stride_b < 0 ||
        h_stride_row < 0 || w_stride_row < K)
        return TMV_ERR_ARG;
    if (B == 0) return TMV_OK;
    if (!tokens || !hidden || !lm_head || !n_nodes || !anc || !depth || !status || !accept_len || !next_token)
        return TMV_ERR_ARG;
    if (D_max > 0 && !path) return TMV_ERR_ARG;
    if (!workspace || workspace_bytes < tmv_tree_accept_lm_head_workspace(B, M_max)) return TMV_ERR_ARG;
    // 16-byte operand loads: aligned bases and strides in whole 8-element groups; byte
    // offsets of every row fit the 32-bit buffer offsets
    if (((reinterpret_cast<uintptr_t>(hidden) | reinterpret_cast<uintptr_t>(lm_head) |
          reinterpret_cast<uintptr_t>(workspace)) & 15u) != 0)
        return TMV_ERR_ARG;
    if (((h_stride_b | h_stride_row | w_stride_row) & 7) != 0) return TMV_ERR_ARG;
    const int64_t h_bytes = ((B - 1) * h_stride_b + static_cast<int64_t>(M_max) * h_stride_row + K) * 2;
    const int64_t w_bytes = (static_cast<int64_t>(V - 1) * w_stride_row + K) * 2;
    if (h_bytes >= (int64_t(1) << 31) || w_bytes >= (int64_t(1) << 31)) return TMV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint64_t *keys = static_cast<uint64_t *>(workspace);
    const int nrows = B * (M_max + 1);
    if (nrows > kLmRows) {
        // more rows than one 64-row block: 272-row blocks against 128-entry tiles
        const int nrb = (nrows + kLwRows - 1) / kLwRows;
        const int ntiles = (V + kLwTile - 1) / kLwTile;
        const int64_t groups = 8ll * nrb * ((ntiles + 7) / 8);
        if (groups > 0x7fffffff) return TMV_ERR_ARG;
        hipLaunchKernelGGL(lm_head_argmax_wide_kernel, dim3(static_cast<unsigned>(groups)), dim3(kLwThreads), 0, s, B,
                           M_max, K, V, static_cast<const uint16_t *>(hidden), h_stride_b, h_stride_row,
                           static_cast<uint32_t>(h_bytes), static_cast<const uint16_t *>(lm_head), w_stride_row,
                           static_cast<uint32_t>(w_bytes), n_nodes, depth, status, keys, ntiles, nrb);
        hipLaunchKernelGGL(lm_select_kernel, dim3(B), dim3(kScanThreads), 0, s, M_max, D_max, V, tokens, n_nodes, anc,
                           depth, status, accept_len, path, next_token, keys, row_argmax);
        return tmv_host::launch_status(hipGetLastError());
    }
    const int nrb = (nrows + kLmRows - 1) / kLmRows;
    const int ntiles = (V + kLmTile - 1) / kLmTile;
    // every workgroup takes kLmTpw tiles of one row block: ntp tile pairs x nrb row blocks,
    // laid out in groups of 8 tile pairs (see the kernel)
    const int ntp = (ntiles + kLmTpw - 1) / kLmTpw;
    const int64_t groups = 8ll * nrb * ((ntp + 7) / 8);
    if (groups > 0x7fffffff) return TMV_ERR_ARG;
#define TMV_LAUNCH_LM(NKS)                                                                                     \
    hipLaunchKernelGGL(lm_head_argmax_kernel<NKS>, dim3(static_cast<unsigned>(groups)), dim3(kLmThreads), 0, s, B,  \
                       M_max, V, static_cast<const uint16_t *>(hidden), h_stride_b, h_stride_row,                  \
                       static_cast<uint32_t>(h_bytes), static_cast<const uint16_t *>(lm_head), w_stride_row,       \
                       static_cast<uint32_t>(w_bytes), n_nodes, depth, status, keys, ntiles, ntp, nrb)
    switch (K) {
    case 512: TMV_LAUNCH_LM(16); break;
    case 1024: TMV_LAUNCH_LM(32); break;
    case 2048: TMV_LAUNCH_LM(64); break;
    case 4096: TMV_LAUNCH_LM(128); break;
    case 8192: TMV_LAUNCH_LM(256); break;
    default: return TMV_ERR_ARG;
    }
#undef TMV_LAUNCH_LM
    hipLaunchKernelGGL(lm_select_kernel, dim3(B), dim3(kScanThreads), 0, s, M_max, D_max, V, tokens, n_nodes, anc,
                       depth, status, accept_len, path, next_token, keys, row_argmax);
    return tmv_host::launch_status(hipGetLastError());
}
