// verify_attention.hip -- tree-masked attention of a flattened draft tree (gfx950).
//
// Every draft node attends to the committed KV prefix plus its own ancestor path,
// itself included, and to nothing else (EAGLE-Pangu, Chinese technical summary section
// 2.3; Medusa section of "Speculative Decoding Hierarquico: Medusa, EAGLE-2 e
// Multi-Token Prediction").  The pages feed a materialised 4D mask to a fused NPU
// kernel; here each query row's ancestor set is a 128-bit mask built in registers from
// the ancestor table, applied only to the <= M tree columns.
//
// bf16, head dim 128 (tree_attn_bf16_kernel):
//   * rows of one KV head = (node, query head in the GQA group), node-major; a workgroup
//     of 8 waves (two per SIMD) owns a row group of 64, 128 or 256 rows and one token
//     split of the (sequence, KV head).  K/V arrive in 32-token chunks through a 128 KiB
//     LDS ring filled by buffer-to-LDS DMA: rounds of 2 (or 4) chunks, up to 3 (or 1)
//     rounds in flight while one is computed, one barrier per round (ring_schedule.hpp);
//     every wave along the rows reads each staged chunk, so a chunk load serves the
//     whole row group.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 leaves each lane holding the scores of ONE
//     query row for 8 tokens, exactly its slice of the B operand of O^T = V^T P^T, so
//     probabilities never move between lanes; V^T operands come from LDS through the
//     transposing ds_read_b64_tr_b16.
//   * softmax in base 2: the query tile carries scale * log2 e and the score MFMAs start
//     from minus a fixed per-row reference (the first finite chunk maximum), so they yield
//     the exponents directly; the split is recomputed against the exact maxima in the rare
//     case a score outgrows the reference by 2^32; row sums come out of the PV product.
//   * token groups of waves share a row group and are combined in LDS at the end; token
//     splits publish (m, l, bf16 rows) and the last split of a row block to arrive merges
//     the block in split order (deterministic).
//   * workgroup ids are laid out so that every workgroup of one (sequence, KV head) lands
//     on the same XCD: the head's K/V goes from HBM into that XCD's L2 once and is re-read
//     by the head's other row groups from there, and the split partials are exchanged
//     through that L2 (plain stores, L1-bypassing loads; a block found spread over several
//     XCDs is rejected, never merged from stale data).
// bf16, head dim 64 (tree_attn_bf16_stream_kernel): 4 waves streaming their chunks straight
//   into registers, split partials merged by tree_attn_merge_kernel.
// fp32 (tree_attn_f32_kernel): one workgroup of 4 waves per (node, query head), the row's
//   64-token chunks dealt to the waves, plain FMA, waves merged in LDS.
#include <cstdlib>
#include <cstdio>
#include <mutex>

#include "tmv_device.hpp"
#include "ring_schedule.hpp"

namespace {

using tmv::kWave;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kOverflow = 32.0f;  // largest score excess over a row's reference, base 2
constexpr int kBufferFlags = 0x00020000;   // raw buffer descriptor word 3 (gfx9 family)

// s_waitcnt immediate that waits for vector-memory count <= N only (gfx9 encoding:
// vmcnt[3:0] and vmcnt[5:4] at bits 15:14, expcnt and lgkmcnt left at their maxima)
template <int N>
constexpr int kVmcntRound() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    return (N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14);
}
constexpr int kVmcntZero = kVmcntRound<0>();
// buffer cache policy sc0: the load misses the CU's own L1 and reads the XCD's L2, where
// every other CU of the XCD has written (L1s write through to the L2)
constexpr int kXcdCoherent = 1;
// s_waitcnt immediate that waits for LDS / scalar-memory count 0 only
constexpr int kLgkmcntZero = 0xF | (0x7 << 4) | (0x3 << 14);

// The ring kernel's two waves per SIMD alternate between MFMA bursts (the score and the PV
// products of a chunk) and VALU / LDS work (softmax, operand reads).  A wave runs its bursts
// at raised priority, so when both waves of a SIMD can issue, the one in its burst goes
// first and the other's VALU work fills the MFMA pipeline's shadow (workload 4 attention
// about 3 %, workload 3 about 5 % faster).  The scheduling barriers keep the compiler from
// moving instructions across the priority changes.
__device__ __forceinline__ void mfma_priority(int p) {
    __builtin_amdgcn_sched_barrier(0);
    if (p) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
}

// LDS accesses outside the ring's chunk loop that run while buffer->LDS copies are in
// flight (the query-tile exchange, the zeroing of V rows past the visible range): the
// compiler cannot tell which LDS bytes a copy in flight writes there, so for an LDS access
// it writes itself it would first wait for every copy.  These are therefore inline
// assembly, each block self-contained: it issues its accesses and waits for them before
// its outputs exist, so no register is ever seen before its data has landed (outputs are
// early-clobber: a returning read must not overwrite a later read's address).  The loop's
// own waits and barriers order the blocks against the copies (the memory clobber keeps the
// compiler from moving them across those).  The chunk operands of 64- and 128-row groups
// are read by such blocks too; 256-row groups read them with ordinary loads, in a loop
// unrolled over the ring groups, each a separate LDS array named statically (the compiler
// then waits only for the copies into the group it reads).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_read_b128_x8(u32x4_t (&v)[8], const uint32_t (&a)[8]) {
    asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
                 "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
                   "=&v"(v[7])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
                 : "memory");
}
// V^T operand reads in inline assembly (see the note above): ds_read_b64_tr_b16 at the
// lane's half offsets z0, z1 with 32*nt XORed in, v[2*nt + h] as in compute_chunk.
__device__ __forceinline__ void lds_read_vt(u32x2_t (&v)[16], uint32_t z0, uint32_t z1) {
    uint32_t t0, t1;
    asm volatile("ds_read_b64_tr_b16 %0, %18\n\t"
                 "ds_read_b64_tr_b16 %1, %19\n\t"
                 "v_xor_b32 %16, 0x20, %18\n\t"
                 "ds_read_b64_tr_b16 %2, %16\n\t"
                 "v_xor_b32 %17, 0x20, %19\n\t"
                 "ds_read_b64_tr_b16 %3, %17\n\t"
                 "v_xor_b32 %16, 0x40, %18\n\t"
                 "ds_read_b64_tr_b16 %4, %16\n\t"
                 "v_xor_b32 %17, 0x40, %19\n\t"
                 "ds_read_b64_tr_b16 %5, %17\n\t"
                 "v_xor_b32 %16, 0x60, %18\n\t"
                 "ds_read_b64_tr_b16 %6, %16\n\t"
                 "v_xor_b32 %17, 0x60, %19\n\t"
                 "ds_read_b64_tr_b16 %7, %17\n\t"
                 "v_xor_b32 %16, 0x80, %18\n\t"
                 "ds_read_b64_tr_b16 %8, %16\n\t"
                 "v_xor_b32 %17, 0x80, %19\n\t"
                 "ds_read_b64_tr_b16 %9, %17\n\t"
                 "v_xor_b32 %16, 0xa0, %18\n\t"
                 "ds_read_b64_tr_b16 %10, %16\n\t"
                 "v_xor_b32 %17, 0xa0, %19\n\t"
                 "ds_read_b64_tr_b16 %11, %17\n\t"
                 "v_xor_b32 %16, 0xc0, %18\n\t"
                 "ds_read_b64_tr_b16 %12, %16\n\t"
                 "v_xor_b32 %17, 0xc0, %19\n\t"
                 "ds_read_b64_tr_b16 %13, %17\n\t"
                 "v_xor_b32 %16, 0xe0, %18\n\t"
                 "ds_read_b64_tr_b16 %14, %16\n\t"
                 "v_xor_b32 %17, 0xe0, %19\n\t"
                 "ds_read_b64_tr_b16 %15, %17\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
                   "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]),
                   "=&v"(v[14]), "=&v"(v[15]), "=&v"(t0), "=&v"(t1)
                 : "v"(z0), "v"(z1)
                 : "memory");
}
// zero 16 bytes of LDS (inline assembly, like the operand reads: a compiler-written LDS
// store would first wait for every buffer->LDS copy in flight)
__device__ __forceinline__ void lds_zero16(uint32_t addr) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(z) : "memory");
}
// store 16 bytes to LDS (inline assembly, for the same reason)
__device__ __forceinline__ void lds_write16(uint32_t addr, u32x4_t v) {
    asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// buffer -> LDS copy of 16 bytes per lane: lane l's bytes land at lds + 16*l; a voffset
// past the descriptor's records writes zeros and reads nothing
__device__ __forceinline__ void dma_to_lds16(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voffset) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voffset, 0, 0, 0);
}
__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char *)p));
}
constexpr int kChunk = 32;          // tokens per chunk (two 16-token MFMA tiles)
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;    // two 16-row tiles

// --------------------------------------------------------------------------- plan
struct AttnPlan {
    int wr;        // waves along rows: d128 ring kernel 2, 4 or 8 of its 8 waves; d64 streaming kernel 1 or 4 of 4
    int rb;        // rows per workgroup = wr * 32
    int nb;        // row blocks per (sequence, kv head)
    int splits;    // token splits per row block
    int pairs;     // B * Hkv
    int per_pair;  // workgroups per pair = nb * splits
    int slots;     // workgroups per XCD (ceil(pairs / 8) * per_pair)
    int adapt;     // ring kernel, ragged batches: one round of this many workgroups (one per CU),
                   // each taking a work item with split counts chosen per sequence on the device
                   // (up to `splits`); 0: off
    int scatter;   // ring kernel: split s of a row block goes to XCD slot (pair + s) % 8 (tests)
};

// split bound of adaptive splitting, and the batch sizes it is used for
constexpr int kAdaptSplits = 2;
constexpr int kAdaptMaxB = 64;

// split-KV row blocks (pairs x row blocks) are limited to the counter block's size (one
// 64-bit arrival word per row block: eight 8-bit counts, one per XCD)
constexpr int kMaxSplitUnits = 4096;
constexpr size_t kCounterBytes = kMaxSplitUnits * sizeof(uint64_t);
// plan flag (ORed into the pinned split count): deal the splits of each row block to
// different XCDs, a placement the L2 partial exchange detects and rejects (tests)
constexpr int kPlanScatter = 0x100;

// An XCD's L2 (4 MB): a (sequence, kv head) pair's K and V rows up to this size stay in
// L2 while the pair's row groups re-read them.
constexpr long kL2Bytes = 4l << 20;

// compute units of the current device (the plan spreads one round of workgroups over them)
int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < tmv::kXcds)
        return 256;
    return cus;
}

// Launch plan.  d128 runs the LDS-ring kernel: 8 waves, two per SIMD, whose 128 KB ring
// keeps one workgroup per CU, so the plan aims for one round of at most `cus` workgroups.
//   * row-group width (rows sharing every staged K/V chunk): the narrowest of 64, 128 and
//     256 rows whose row blocks leave at least four token splits per block within the
//     round; 256 rows when a pair's K/V are larger than an L2 (each row group then
//     re-reads them from HBM, so the rows sharing a chunk load are maximised);
//   * token splits: the most that keep the grid within one round (1 to 16, and at least
//     two chunks for each token group of waves in each split).
// d64 runs the streaming kernel (4 waves, no ring) with 128-row groups from 256 rows on
// and enough splits to reach 256 workgroups.
// `force_rows` / `force_splits` (0 = the rule's choice) pin the plan (tuning and tests).
AttnPlan make_plan(int B, int M_max, int Hq, int Hkv, int L_cap, int d, int cus, int force_rows = 0,
                   int force_splits = 0) {
    AttnPlan p;
    p.scatter = (force_splits & kPlanScatter) ? 1 : 0;
    force_splits &= ~kPlanScatter;
    const int g = Hq / Hkv;
    const int rows = M_max * g;
    p.pairs = B * Hkv;
    // pairs per XCD: workgroup i runs on XCD i % 8 and the grid gives each XCD its own pairs
    const long xcd_pairs = (static_cast<long>(p.pairs) + tmv::kXcds - 1) / tmv::kXcds;
    const long cpx = cus / tmv::kXcds;
    auto blocks = [&](int wr) { return rows > 0 ? (rows + wr * kRowsPerWave - 1) / (wr * kRowsPerWave) : 0; };
    if (d == 128) {
        const long kv_pair = static_cast<long>(L_cap) * d * 2 * 2;
        if (kv_pair > kL2Bytes) p.wr = 8;
        else if (xcd_pairs * blocks(2) * 4 <= cpx) p.wr = 2;
        else if (xcd_pairs * blocks(4) * 4 <= cpx) p.wr = 4;
        else p.wr = 8;
        if (force_rows == 64 || force_rows == 128 || force_rows == 256) p.wr = force_rows / kRowsPerWave;
    } else {
        p.wr = rows >= 256 ? 4 : 1;
        if (force_rows == 32 || force_rows == 128) p.wr = force_rows / kRowsPerWave;
    }
    p.rb = p.wr * kRowsPerWave;
    p.nb = blocks(p.wr);
    const long base = static_cast<long>(p.pairs) * p.nb;
    int s;
    if (d == 128) {
        const int tw = 8 / p.wr;                                     // token groups of waves
        s = base <= 0 ? 1 : static_cast<int>(cpx / (xcd_pairs * p.nb));
        const int s_tok = L_cap / (tw * 2 * kChunk);                 // >= 2 chunks per token group
        if (s > s_tok) s = s_tok;
    } else {
        s = base <= 0 ? 1 : static_cast<int>((256 + base - 1) / base);
        const int s_tok = L_cap / ((kWaves / p.wr) * 2 * kChunk);
        if (s > s_tok) s = s_tok;
    }
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    if (force_splits >= 1 && force_splits <= 16) s = force_splits;
    if (base >= kMaxSplitUnits) s = 1;
    // a ragged batch whose row blocks fit one workgroup per CU but leave no room for uniform
    // splits: the device gives the sequences with the most chunks a second split
    p.adapt = 0;
    if (d == 128 && force_rows == 0 && force_splits == 0 && s == 1 && B >= 2 && B <= kAdaptMaxB &&
        Hkv % tmv::kXcds == 0 && base <= cpx * tmv::kXcds && base < kMaxSplitUnits && L_cap >= 4 * kChunk) {
        p.adapt = static_cast<int>(cpx) * tmv::kXcds;           // one workgroup per CU
        s = kAdaptSplits;
    }
    p.splits = s;
    p.per_pair = p.nb * p.splits;
    p.slots = static_cast<int>(xcd_pairs) * p.per_pair;
    return p;
}

// workspace layout: [arrival counters: kMaxSplitUnits int32][stats: pairs*nb*S*rb*2 f32]
// [partial O: pairs*nb*S*rb*d, bf16 for d128 (normalised rows), f32 for d64 (unnormalised)]
// (the last two only with split-KV).  The counter block sits at the same place for every
// shape and nothing else is ever written there: it must be zero before the first call,
// and every call leaves the counters it used at zero, so a zero-filled workspace stays
// valid across calls of any shape it is large enough for.  Split-KV is only planned for
// fewer than kMaxSplitUnits row blocks (with that many, one split per block already fills
// the chip).
size_t plan_bytes(const AttnPlan &p, int d, size_t *off_o, size_t *off_stats = nullptr) {
    const size_t units = static_cast<size_t>(p.pairs) * p.nb * p.splits * p.rb;
    size_t st = p.splits > 1 ? units * 2 * sizeof(float) : 0;
    st = (st + 255) / 256 * 256;
    const size_t es = d == 128 ? 2 : 4;
    const size_t o = p.splits > 1 ? units * d * es : 0;
    if (off_stats) *off_stats = kCounterBytes;
    if (off_o) *off_o = kCounterBytes + st;
    return kCounterBytes + st + o;
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(p));
}

// --------------------------------------------------------------------------- split merge
// Row rr, dims part*8 .. +8 of split-KV unit `unit`: the S partials (m, l, unnormalised O)
// are read in split order, rescaled to the common maximum and written as the bf16 row;
// rows of inert nodes (and whole failed sequences) are written as 0.
template <int D, int RB>
__device__ __forceinline__ void merge_row_part(int64_t unit, int rr, int part, int splits, int b, int kvh, int g,
                                               int r, int M_max, int L_cap, int M, int P, int st,
                                               const int32_t *__restrict__ depth, uint16_t *__restrict__ out,
                                               int64_t os0, int64_t os1, int64_t os2,
                                               const float *__restrict__ ws_stats, const float *__restrict__ ws_o)
{
    if (r >= M_max * g) return;
    const int j = r / g + 1, gi = r % g;
    const int dp = depth[static_cast<int64_t>(b) * (M_max + 1) + j];
    // every split's (m, l) and O slice are fetched before any is consumed
    constexpr int kMaxSplits = 16;
    float2 ml[kMaxSplits];
    float4 oa[kMaxSplits], ob[kMaxSplits];
#pragma unroll
    for (int s2 = 0; s2 < kMaxSplits; ++s2) {
        if (s2 < splits) {
            const int64_t base = (unit * splits + s2) * RB + rr;
            ml[s2] = *reinterpret_cast<const float2 *>(ws_stats + base * 2);
            const float4 *o = reinterpret_cast<const float4 *>(ws_o + base * D + part * 8);
            oa[s2] = o[0];
            ob[s2] = o[1];
        }
    }
    const bool seq_ok = st == TMV_OK && M >= 0 && M <= M_max && P >= 0 && static_cast<int64_t>(P) + M <= L_cap;
    const bool live = seq_ok && r < M * g && dp >= 1;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (live) {
        float mt = -INFINITY;
#pragma unroll
        for (int s2 = 0; s2 < kMaxSplits; ++s2)
            if (s2 < splits) mt = fmaxf(mt, ml[s2].x);
        const float mref = mt == -INFINITY ? 0.f : mt;
        float lt = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < kMaxSplits; ++s2) {
            if (s2 < splits) {
                const float sc = __builtin_amdgcn_exp2f(ml[s2].x - mref);
                lt += sc * ml[s2].y;
                acc[0] += sc * oa[s2].x; acc[1] += sc * oa[s2].y; acc[2] += sc * oa[s2].z; acc[3] += sc * oa[s2].w;
                acc[4] += sc * ob[s2].x; acc[5] += sc * ob[s2].y; acc[6] += sc * ob[s2].z; acc[7] += sc * ob[s2].w;
            }
        }
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= inv;
    }
    uint32_t w4[4];
#pragma unroll
    for (int h2 = 0; h2 < 4; ++h2)
        w4[h2] = static_cast<uint32_t>(tmv::f32_to_bf16(acc[2 * h2])) |
                 (static_cast<uint32_t>(tmv::f32_to_bf16(acc[2 * h2 + 1])) << 16);
    uint16_t *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + static_cast<int64_t>(kvh * g + gi) * os2 + part * 8;
    *reinterpret_cast<uint4 *>(o) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
}

// One thread per (row, 8 head dims) of every live row block (the register-streaming
// kernel's split-KV merge, ordered after it on the stream).
template <int D, int RB>
__global__ void __launch_bounds__(256)
tree_attn_merge_kernel(int M_max, int D_max, int Hq, int Hkv, int L_cap,
                       const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
                       const int32_t *__restrict__ depth, const int32_t *__restrict__ status,
                       uint16_t *__restrict__ out, int64_t os0, int64_t os1, int64_t os2,
                       const float *__restrict__ ws_stats, const float *__restrict__ ws_o,
                       int pairs, int nb, int splits)
{
    constexpr int TPR = D / 8;                         // threads per row
    const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
    const int64_t row_global = t / TPR;                // over pairs * nb * RB
    const int part = static_cast<int>(t % TPR);
    if (row_global >= static_cast<int64_t>(pairs) * nb * RB) return;
    const int64_t unit = row_global / RB;
    const int rr = static_cast<int>(row_global % RB);
    const int pair = static_cast<int>(unit / nb), rbk = static_cast<int>(unit % nb);
    const int b = pair / Hkv, kvh = pair % Hkv, g = Hq / Hkv;
    merge_row_part<D, RB>(unit, rr, part, splits, b, kvh, g, rbk * RB + rr, M_max, L_cap, n_nodes[b], prefix_len[b],
                          status[b], depth, out, os0, os1, os2, ws_stats, ws_o);
}

// ------------------------------------------------ bf16 MFMA kernel, register streaming (d64)
// Each wave streams its own chunks straight from memory into registers; used for head
// dimension 64, where the LDS-ring kernel below is switched off.
template <int D, int WR>
__global__ void __launch_bounds__(kWaves * kWave)
tree_attn_bf16_stream_kernel(int M_max, int D_max, int Hq, int Hkv,
                      const uint16_t *__restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
                      const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
                      int64_t ks0, int64_t ks1, int64_t ks2, int L_cap,
                      const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
                      const int32_t *__restrict__ anc, const int32_t *__restrict__ depth,
                      int32_t *__restrict__ status, float qk_scale_log2,
                      uint16_t *__restrict__ out, int64_t os0, int64_t os1, int64_t os2,
                      float *__restrict__ ws_stats, float *__restrict__ ws_o,
                      int pairs, int nb, int splits, int per_pair)
{
    constexpr int KS = D / 32;           // k-steps of the QK^T contraction
    constexpr int NT = D / 16;           // 16-dim output tiles
    constexpr int WT = kWaves / WR;      // waves sharing rows (token split inside the WG)
    constexpr int RB = WR * kRowsPerWave;
    constexpr int DG = D / 4;            // dims per lane of an output row

    // ---- decode the workgroup: XCD-major so one (sequence, kv head) stays on one XCD
    const int wg = blockIdx.x;
    const int xcd = wg % tmv::kXcds, slot = wg / tmv::kXcds;
    const int pair = (slot / per_pair) * tmv::kXcds + xcd;
    if (pair >= pairs) return;
    const int within = slot % per_pair;
    const int rbk = within / splits, split = within % splits;
    const int b = pair / Hkv, kvh = pair % Hkv;
    const int g = Hq / Hkv;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);     // wave-uniform
    const int wr = wave / WT, wt = wave % WT;
    const int c16 = lane & 15, G = lane >> 4;
    auto row0_of = [&](int rb_, int wr_) { return rb_ * RB + wr_ * kRowsPerWave; };

    const int R = 1 + M_max, W = D_max + 1;
    constexpr int kAncBatch = 8;                           // ancestor entries fetched up front

    // ---- one round trip for everything the prologue needs: the sequence's scalars and,
    // independently of them, this lane's query fragments, node depths and first ancestor
    // entries (row indices are clamped into the tables, so no load waits on another)
    const int M = n_nodes[b];
    const int P = prefix_len[b];
    int st = status[b];
    bf16x8_t qf[2][KS];
    int dep[2], anc8[2][kAncBatch];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        int r = row0_of(rbk, wr) + rt * 16 + c16;
        if (r > M_max * g - 1) r = M_max * g - 1;
        const int j = r / g + 1, gi = r % g;
        const uint16_t *qp = q + b * qs0 + static_cast<int64_t>(j - 1) * qs1 + static_cast<int64_t>(kvh * g + gi) * qs2 + G * 8;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = load_bf16x8(qp + ks * 32);
        dep[rt] = depth[static_cast<int64_t>(b) * R + j];
        const int32_t *arow = anc + (static_cast<int64_t>(b) * R + j) * W;
#pragma unroll
        for (int k = 0; k < kAncBatch; ++k) anc8[rt][k] = arow[k < W ? k : W - 1];
    }

    if (st == TMV_OK && (M < 0 || M > M_max || P < 0 || static_cast<int64_t>(P) + M > L_cap)) {
        st = TMV_ERR_INPUT;
        if (threadIdx.x == 0 && rbk == 0 && split == 0) status[b] = TMV_ERR_INPUT;
    }
    const int Rh = (st == TMV_OK) ? M * g : 0;           // live rows of this kv head
    const int row0_wg = rbk * RB;
    const int row0 = row0_wg + wr * kRowsPerWave;         // first row of this wave

    // rows of this wave: r = row0 + rt*16 + c16 (lane's row in each tile)
    auto write_zero_rows = [&](int first) {
        // the wave's 32 rows: each lane clears dims G*DG .. +DG of its row in each tile
        for (int rt = 0; rt < 2; ++rt) {
            const int r = first + rt * 16 + c16;
            if (r >= M_max * g) continue;
            const int j = r / g + 1, gi = r % g;
            uint16_t *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + static_cast<int64_t>(kvh * g + gi) * os2 + G * DG;
#pragma unroll
            for (int e = 0; e < DG; e += 8) *reinterpret_cast<uint4 *>(o + e) = make_uint4(0, 0, 0, 0);
        }
    };

    if (row0_wg >= Rh) {
        // no live row in this workgroup: clear the block's output rows (with split-KV the
        // merge kernel writes every row instead)
        if (splits == 1 && wt == 0) write_zero_rows(row0);
        return;
    }
    const bool wave_live = row0 < Rh;

    // query fragments live in LDS (one copy per row group) rather than in 2*KS*4 VGPRs;
    // each chunk reads them back with 16-byte LDS loads in lane order (conflict-free)
    __shared__ uint4 q_lds[WR][2][KS][kWave];
    if (wt == 0) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) q_lds[wr][rt][ks][lane] = __builtin_bit_cast(uint4, qf[rt][ks]);
    }
    __syncthreads();

    // ---- ancestor-or-self masks of the lane's two rows (bit a <-> tree slot P + a);
    // rows beyond the live ones are padding whose results are never written
    uint64_t mlo[2] = {0, 0}, mhi[2] = {0, 0};
    const int T = P + M;                                  // tokens visible to someone
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = row0 + rt * 16 + c16;
        if (r >= Rh) continue;
        const int dp = dep[rt];
#pragma unroll
        for (int k = 0; k < kAncBatch; ++k)
            if (k < dp) {
                const int a = anc8[rt][k] - 1;
                if (a < 64) mlo[rt] |= 1ull << a; else mhi[rt] |= 1ull << (a - 64);
            }
        if (dp > kAncBatch) {
            const int j = r / g + 1;
            const int32_t *arow = anc + (static_cast<int64_t>(b) * R + j) * W;
            for (int k = kAncBatch; k < dp; ++k) {
                const int a = arow[k] - 1;
                if (a < 64) mlo[rt] |= 1ull << a; else mhi[rt] |= 1ull << (a - 64);
            }
        }
    }

    // ---- token range of this split (in chunks), interleaved over the WT waves
    const int nchunks = (T + kChunk - 1) / kChunk;
    const int c_begin = static_cast<int>(static_cast<int64_t>(nchunks) * split / splits);
    const int c_end = static_cast<int>(static_cast<int64_t>(nchunks) * (split + 1) / splits);

    // chunk addressing: buffer loads through a wave-uniform resource descriptor rebuilt
    // per chunk (scalar ALU only) plus per-lane byte offsets that never change.  The
    // descriptor's record count stops at token T, so loads past the sequence return 0
    // and never touch memory outside it.  K fragment (tt, ks) of a lane: token
    // tt*16 + c16, dims ks*32 + G*8 .. +8 (the four lane groups of one instruction cover
    // 64 contiguous bytes of a row); V row jj of a lane: token pi(G*8 + jj), dims
    // c16*NT .. +NT (16 lanes cover a whole row).
    const char *kbase = reinterpret_cast<const char *>(kc + b * ks0 + kvh * ks1);
    const char *vbase = reinterpret_cast<const char *>(vc + b * ks0 + kvh * ks1);
    const int64_t row_bytes = ks2 * 2;
    uint32_t offk[2], offv[8];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) offk[tt] = static_cast<uint32_t>((tt * 16 + c16) * row_bytes + G * 16);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
        offv[jj] = static_cast<uint32_t>((jj < 4 ? G * 4 + jj : 16 + G * 4 + (jj - 4)) * row_bytes + c16 * NT * 2);

    f32x4_t oacc[2][NT];
    float mref[2], mtrue[2], lrow[2];
    const float cs = qk_scale_log2;

    struct Chunk {
        bf16x8_t kf[2][KS];
        uint4 vr[8];
    };
    auto load_chunk = [&](Chunk &ch, int c) {
        const int t0 = c * kChunk;
        const int64_t left = static_cast<int64_t>(T - t0) * row_bytes;
        const int records = static_cast<int>(left < 0 ? 0 : (left > kChunk * row_bytes ? kChunk * row_bytes : left));
        __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(kbase + t0 * row_bytes), 0, records, kBufferFlags);
        __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(vbase + t0 * row_bytes), 0, records, kBufferFlags);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                ch.kf[tt][ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(kr, offk[tt] + ks * 64, 0, 0));
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            if constexpr (NT == 8) {
                ch.vr[jj] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vrs, offv[jj], 0, 0));
            } else {
                const auto u = __builtin_amdgcn_raw_buffer_load_b64(vrs, offv[jj], 0, 0);
                ch.vr[jj] = make_uint4(u[0], u[1], 0, 0);
            }
        }
    };
    auto xor16_max = [](float x) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    auto xor32_max = [](float x) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    // first pass: each row's reference is the first finite chunk maximum (O and l are
    // still exactly zero then, so adopting it rescales nothing); later maxima are only
    // tracked.  p = 2^(s*cs - ref) stays finite unless a score exceeds the reference by
    // more than kOverflow in base 2, in which case the whole split is recomputed against
    // the exact maximum -- the accumulators never need rescaling inside the loop.
    bool first_pass = true, overflow = false;
    auto compute_chunk = [&](const Chunk &ch, int c) {
        const int t0 = c * kChunk;
        // S^T tiles: [token][row]; lane holds row c16 of tile rt, tokens t0 + tt*16 + G*4 + i
        f32x4_t s[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            bf16x8_t qr[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qr[ks] = __builtin_bit_cast(bf16x8_t, q_lds[wr][rt][ks][lane]);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.kf[tt][ks], qr[ks], acc, 0, 0, 0);
                s[rt][tt] = acc;
            }
        }
        if (t0 + kChunk > P) {
            // chunk reaches the tree slots: a token is visible if it is in the prefix or
            // is an ancestor-or-self of the row's node (bit t - P of the row's mask)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int a = t0 + tt * 16 + G * 4 + i - P;
                        const uint64_t word = a >= 64 ? mhi[rt] : mlo[rt];
                        const bool bit = (word >> (a & 63)) & 1ull;
                        const bool vis = a < 0 || (a < M && bit);
                        s[rt][tt][i] = vis ? s[rt][tt][i] : -INFINITY;
                    }
        }
        bf16x8_t pb[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            if (first_pass) {
                float cm = fmaxf(fmaxf(fmaxf(s[rt][0][0], s[rt][0][1]), fmaxf(s[rt][0][2], s[rt][0][3])),
                                 fmaxf(fmaxf(s[rt][1][0], s[rt][1][1]), fmaxf(s[rt][1][2], s[rt][1][3])));
                cm = xor32_max(xor16_max(cm));
                mtrue[rt] = fmaxf(mtrue[rt], cm);
                if (mref[rt] == -INFINITY) mref[rt] = cm;
                overflow |= (cm - mref[rt]) * cs > kOverflow;
            }
            const float mr = mref[rt] == -INFINITY ? 0.f : mref[rt] * cs;
            float lsum = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rt][tt][i], cs, -mr));
                    pb[rt][tt * 4 + i] = static_cast<__bf16>(pe);
                    lsum += pe;
                }
            lrow[rt] += lsum;
        }
        // O^T += V^T P^T; A operand of dim tile nt = (vr[0][nt], ..., vr[7][nt])
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint32_t a4[4];
            const uint32_t sel = (nt & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint4 x4 = ch.vr[2 * f], y4 = ch.vr[2 * f + 1];
                const int e = nt >> 1;
                const uint32_t x = e == 0 ? x4.x : e == 1 ? x4.y : e == 2 ? x4.z : x4.w;
                const uint32_t y = e == 0 ? y4.x : e == 1 ? y4.y : e == 2 ? y4.z : y4.w;
                a4[f] = __builtin_amdgcn_perm(y, x, sel);
            }
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a4[0], a4[1], a4[2], a4[3]));
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                oacc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], oacc[rt][nt], 0, 0, 0);
        }
    };

#pragma unroll
    for (int rt = 0; rt < 2; ++rt) { mref[rt] = -INFINITY; mtrue[rt] = -INFINITY; }
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            lrow[rt] = 0.f;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) oacc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (wave_live) {
            // ping-pong register buffers: the next chunk's loads are in flight while the
            // current chunk is computed (the prefetch index is clamped into the range)
            Chunk bufA, bufB;
            int c = c_begin + wt;
            if (c < c_end) load_chunk(bufA, c);
            while (c < c_end) {
                const int c1 = c + WT;
                load_chunk(bufB, c1 < c_end ? c1 : c);
                compute_chunk(bufA, c);
                if (c1 >= c_end) break;
                const int c2 = c1 + WT;
                load_chunk(bufA, c2 < c_end ? c2 : c1);
                compute_chunk(bufB, c1);
                c = c2;
            }
        }
        if (!__any(overflow)) break;
        // rare: some score outgrew its reference; redo the split against the exact maxima
        first_pass = false;
        overflow = false;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) mref[rt] = mtrue[rt];
    }
    float mrow[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        mrow[rt] = mref[rt];
        // row sums: each of the four lanes of a row holds a partial sum
        auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lrow[rt]), __float_as_uint(lrow[rt]), false, false);
        const float l16 = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
        auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l16), __float_as_uint(l16), false, false);
        lrow[rt] = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
    }
    // from here on the running maxima are in base-2 units, as the merge steps expect
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) mrow[rt] = mrow[rt] == -INFINITY ? -INFINITY : mrow[rt] * cs;

    // ---- merge the WT waves that share rows (LDS), fixed order
    // lane's output element (rt, nt, i) is row row0 + rt*16 + c16, dim (G*4 + i)*NT + nt
    if constexpr (WT > 1) {
        __shared__ float lds_o[(WT - 1) * kRowsPerWave * D];
        __shared__ float lds_ml[(WT - 1) * kRowsPerWave * 2];
        if (wt > 0) {
            float *o = lds_o + (wt - 1) * kRowsPerWave * D;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int rr = rt * 16 + c16;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[rr * D + (G * 4 + i) * NT + nt] = oacc[rt][nt][i];
                if (G == 0) {
                    lds_ml[((wt - 1) * kRowsPerWave + rr) * 2 + 0] = mrow[rt];
                    lds_ml[((wt - 1) * kRowsPerWave + rr) * 2 + 1] = lrow[rt];
                }
            }
        }
        __syncthreads();
        if (wt == 0) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int rr = rt * 16 + c16;
                float mo[WT], lo_[WT];
                mo[0] = mrow[rt]; lo_[0] = lrow[rt];
                float mt = mo[0];
#pragma unroll
                for (int w = 1; w < WT; ++w) {
                    mo[w] = lds_ml[((w - 1) * kRowsPerWave + rr) * 2 + 0];
                    lo_[w] = lds_ml[((w - 1) * kRowsPerWave + rr) * 2 + 1];
                    mt = fmaxf(mt, mo[w]);
                }
                const float mref = mt == -INFINITY ? 0.f : mt;
                float sc[WT], lt = 0.f;
#pragma unroll
                for (int w = 0; w < WT; ++w) { sc[w] = __builtin_amdgcn_exp2f(mo[w] - mref); lt += sc[w] * lo_[w]; }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float acc = oacc[rt][nt][i] * sc[0];
#pragma unroll
                        for (int w = 1; w < WT; ++w)
                            acc += sc[w] * lds_o[(w - 1) * kRowsPerWave * D + rr * D + (G * 4 + i) * NT + nt];
                        oacc[rt][nt][i] = acc;
                    }
                mrow[rt] = mt;
                lrow[rt] = lt;
            }
        }
    }

    // ---- split-KV: publish this split's partial (m, l, unnormalised O) and stop; the
    // merge kernel that follows on the stream combines the splits in a fixed order
    if (splits > 1) {
        if (wt != 0) return;
        const int64_t unit = static_cast<int64_t>(pair) * nb + rbk;          // (pair, row block)
        const int64_t base = (unit * splits + split) * RB + wr * kRowsPerWave;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int rr = rt * 16 + c16;
            float *o = ws_o + (base + rr) * D + G * DG;
#pragma unroll
            for (int e = 0; e < DG; e += 4) {
                float4 v4;
                v4.x = oacc[rt][(e + 0) % NT][(e + 0) / NT];
                v4.y = oacc[rt][(e + 1) % NT][(e + 1) / NT];
                v4.z = oacc[rt][(e + 2) % NT][(e + 2) / NT];
                v4.w = oacc[rt][(e + 3) % NT][(e + 3) / NT];
                *reinterpret_cast<float4 *>(o + e) = v4;
            }
            if (G == 0) *reinterpret_cast<float2 *>(ws_stats + (base + rr) * 2) = make_float2(mrow[rt], lrow[rt]);
        }
        return;
    }
    if (wt != 0) return;

    // ---- write the final rows: lane writes dims G*DG .. +DG of its row in each tile
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = row0 + rt * 16 + c16;
        if (r >= M_max * g) continue;
        const int j = r / g + 1, gi = r % g;
        const bool live = r < Rh && depth[static_cast<int64_t>(b) * R + j] >= 1;
        const float inv = live && lrow[rt] > 0.f ? 1.f / lrow[rt] : 0.f;
        uint16_t *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + static_cast<int64_t>(kvh * g + gi) * os2 + G * DG;
#pragma unroll
        for (int e = 0; e < DG; e += 8) {
            uint32_t w4[4];
#pragma unroll
            for (int h2 = 0; h2 < 4; ++h2) {
                // dims e + 2*h2, e + 2*h2 + 1 of this lane's slice: (i, nt) = (dim / NT, dim % NT)
                const int d0 = e + 2 * h2, d1 = d0 + 1;
                const float x0 = live ? oacc[rt][d0 % NT][d0 / NT] * inv : 0.f;
                const float x1 = live ? oacc[rt][d1 % NT][d1 / NT] * inv : 0.f;
                w4[h2] = tmv::pack_bf16x2(x0, x1);
            }
            *reinterpret_cast<uint4 *>(o + e) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
    }
}

// --------------------------------------------------------------------------- bf16 MFMA kernel (d128)
// LDS ring of chunk slots: 128 KiB, two halves of kRound chunks each (double buffered).
constexpr int kRingBytes = 128 * 1024;
constexpr int kRingWaves = 8;       // waves of the ring kernel: two per SIMD

template <int D>
struct RingShape {
    static constexpr int kRowBytes = D * 2;                 // one K (or V) row in LDS
    static constexpr int kPieces = D / 8;                   // 16-byte pieces per row
    static constexpr int kMatBytes = kChunk * kRowBytes;    // K (or V) part of one chunk
    static constexpr int kSlotBytes = 2 * kMatBytes;        // K then V
    static constexpr int kSlots = kRingBytes / kSlotBytes;  // 8 (d128)
    static constexpr int kDmaPerChunk = kSlotBytes / 1024;  // 1 KiB per DMA instruction
    static constexpr int kDmaPerWave = kDmaPerChunk / kRingWaves;
    static_assert(kDmaPerWave * kRingWaves == kDmaPerChunk, "chunk DMA must split evenly over the waves");
};

// ancestor entries of a row fetched in the prologue (four per lane); deeper rows (DEEP
// kernels only) fetch the rest in further batches
constexpr int kAncBatch = 16;

// paged caches: block-table entries of one sequence staged in LDS (the ring leaves 32 KB)
constexpr int kMaxPagesLds = 4096;

// block table of a paged cache (PAGED kernels): page of logical token t of sequence b is
// tab[b * stride + (t >> shift)], valid when in [0, npages)
struct PagedArgs {
    const int32_t *tab;
    int64_t stride;
    int shift;
    int npages;
};

// The merging workgroup of a split-KV row block (LDS-ring kernel).  Split s left, per row
// of the block, (m, l) in fp32 -- m the row's largest score in base-2 units, l the sum of
// 2^(score - m) -- and the row's output normalised by l, rounded to bf16.  Every (split,
// row) statistic is loaded once and shared through LDS (lds_ml, RB * SMAX pairs); a thread
// merges items (row rr, dims part*8 .. +8), two at a time: the rows' depths and every
// split's 16-byte O slice of those items are loaded in one straight batch (the first batch
// right after the statistics, so these are staged while it travels), then merged in split
// order, so the result does not depend on which split arrived last.  The partials were
// written by the block's other workgroups on this XCD with plain stores, so they sit in its
// L2: the loads skip the L1 and read them there.  The buffer descriptors end at the
// `splits`-th partial: loads of splits past it return zeros without touching memory and are
// left out of the merge.
template <int D, int RB, int SMAX>
__device__ __forceinline__ void merge_block(int64_t unit, int splits, int stride, int b, int kvh, int g, int g_magic,
                                            int row0_wg, int M_max, int L_cap, int M, int P, int st,
                                            const int32_t *__restrict__ depth, uint16_t *__restrict__ out,
                                            int64_t os0, int64_t os1, int64_t os2, const float *__restrict__ ws_stats,
                                            const uint16_t *__restrict__ ws_o, float *__restrict__ lds_ml)
{
    constexpr int kThreads = kRingWaves * kWave;
    constexpr int kItems = RB * (D / 8);
    static_assert(kItems % kThreads == 0, "whole items per thread");
    constexpr int kIpt = kItems / kThreads;            // items per thread
    constexpr int kPairs = RB * SMAX;                  // (split, row) statistics of the block
    static_assert(kPairs % kThreads == 0, "whole statistics per thread");
    constexpr int kPpt = kPairs / kThreads;
    const __amdgpu_buffer_rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(ws_stats + unit * stride * RB * 2), 0, splits * RB * 2 * 4, kBufferFlags);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(ws_o + unit * stride * RB * D), 0, splits * RB * D * 2, kBufferFlags);
    const bool seq_ok = st == TMV_OK && M >= 0 && M <= M_max && P >= 0 && static_cast<int64_t>(P) + M <= L_cap;
    const int rows_max = M_max * g;
    const int tid = static_cast<int>(threadIdx.x);
    // pair i*kThreads + tid is (split, row) = (pidx / RB, pidx % RB): the partials' own order
    u32x2_t mlp[kPpt];
#pragma unroll
    for (int i = 0; i < kPpt; ++i) mlp[i] = __builtin_amdgcn_raw_buffer_load_b64(rst, (i * kThreads + tid) * 8, 0, kXcdCoherent);
    // items in batches of IPB per thread: the rows' depths and every split's O slices
    constexpr int IPB = kIpt < 2 ? kIpt : 2;
    u32x4_t ov[IPB][SMAX];
    int dp[IPB];
    auto load_batch = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < IPB; ++k) {
            const int item = (i0 + k) * kThreads + tid;
            const int rr = item / (D / 8), part = item % (D / 8);
            int r = row0_wg + rr;
            r = r < rows_max ? r : rows_max - 1;
            dp[k] = depth[static_cast<int64_t>(b) * (M_max + 1) + ((r * g_magic) >> 16) + 1];
#pragma unroll
            for (int s2 = 0; s2 < SMAX; ++s2)
                ov[k][s2] = __builtin_amdgcn_raw_buffer_load_b128(ro, ((s2 * RB + rr) * D + part * 8) * 2, 0, kXcdCoherent);
        }
    };
    load_batch(0);
    // the statistics, row-major ([row][split]) in LDS, while the first batch travels
#pragma unroll
    for (int i = 0; i < kPpt; ++i) {
        const int pidx = i * kThreads + tid, s2 = pidx / RB, rr = pidx % RB;
        *reinterpret_cast<u32x2_t *>(lds_ml + (rr * SMAX + s2) * 2) = mlp[i];
    }
    __syncthreads();
#pragma unroll 1
    for (int i0 = 0; i0 < kIpt; i0 += IPB) {
        if (i0 > 0) load_batch(i0);
#pragma unroll
        for (int k = 0; k < IPB; ++k) {
            const int item = (i0 + k) * kThreads + tid;
            const int rr = item / (D / 8), part = item % (D / 8);
            const int r = row0_wg + rr;
            float2 ml[SMAX];
#pragma unroll
            for (int s2 = 0; s2 < SMAX; s2 += 2) {
                const float4 x = *reinterpret_cast<const float4 *>(lds_ml + (rr * SMAX + s2) * 2);
                ml[s2] = make_float2(x.x, x.y);
                ml[s2 + 1] = make_float2(x.z, x.w);
            }
            float mt = -INFINITY;
#pragma unroll
            for (int s2 = 0; s2 < SMAX; ++s2)
                if (s2 < splits) mt = fmaxf(mt, ml[s2].x);
            const float mref = mt == -INFINITY ? 0.f : mt;
            float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float lt = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < SMAX; ++s2) {
                // weight of split s2: its share of the row's softmax mass (0 past the splits)
                const float w = s2 < splits ? __builtin_amdgcn_exp2f(ml[s2].x - mref) * ml[s2].y : 0.f;
                lt += w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[2 * e] += w * __uint_as_float(ov[k][s2][e] << 16);
                    acc[2 * e + 1] += w * __uint_as_float(ov[k][s2][e] & 0xffff0000u);
                }
            }
            // inert rows are zeros whatever their partials hold (computed for every item, live
            // or not, and selected at the end: a branch on liveness would let the compiler sink
            // the partial loads behind the depth load)
            const bool live = seq_ok && r < M * g && dp[k] >= 1;
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
            uint32_t w4[4];
#pragma unroll
            for (int h2 = 0; h2 < 4; ++h2) w4[h2] = live ? tmv::pack_bf16x2(acc[2 * h2] * inv, acc[2 * h2 + 1] * inv) : 0u;
            if (r >= rows_max) continue;
            const int j = ((r * g_magic) >> 16) + 1, gi = r - (j - 1) * g;
            uint16_t *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + static_cast<int64_t>(kvh * g + gi) * os2 + part * 8;
            *reinterpret_cast<uint4 *>(o) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
    }
}

// Tree attention of one (sequence, KV head, row block, token split).  8 waves, two per
// SIMD (at most 256 registers per lane), so one wave's MFMAs overlap the other's softmax
// and LDS reads.  RW waves lie along the rows (RB = 32 RW rows share every staged chunk)
// and TW = 8 / RW token groups of waves take turns on the chunks of each ring round.
// Work item of workgroup w when the splits adapt to a ragged batch (B <= 64 sequences, Hkv a
// multiple of 8; one workgroup per CU, all in one round).  Workgroup w serves XCD slot
// x = w % 8 (KV heads x, x + 8, ...) and takes item w / 8 of that slot.  Each sequence c has
// n_c = max(1, live row groups) row groups per head and s_c = min(smax, ceil(chunks_c / T))
// splits, with the smallest bound T (of 64 candidates, at least two chunks per token group of
// a split) for which every slot's items -- (head, row group, split) of every sequence, in
// sequence order -- fit its gridDim.x / 8 workgroups.  Every workgroup derives the same items
// from the same inputs: the prefix lengths and node counts, which the kernel never writes.
struct AdaptItem {
    int pair, rbk, split, splits;   // pair < 0: no item
    int tail_from;                  // the item that clears the sequence's rows from this row on (-1: none)
};
__device__ __forceinline__ AdaptItem adaptive_item(const int32_t *__restrict__ prefix_len,
                                                   const int32_t *__restrict__ n_nodes, int B, int Hkv, int g, int RB,
                                                   int TW, int M_max, int L_cap, int smax) {
    const int lane = threadIdx.x & (kWave - 1);
    int ch = 0, nbl = 0;                   // lane c: sequence c's chunks and row groups
    if (lane < B) {
        nbl = 1;
        const int P = prefix_len[lane], M = n_nodes[lane];
        if (M >= 0 && M <= M_max && P >= 0 && static_cast<int64_t>(P) + M <= L_cap) {
            ch = (P + M + kChunk - 1) / kChunk;
            const int n = (M * g + RB - 1) / RB;
            nbl = n > 1 ? n : 1;
        }
    }
    int maxc = 0;
    for (int c = 0; c < B; ++c) {
        const int x = __builtin_amdgcn_readlane(ch, c);
        maxc = x > maxc ? x : maxc;
    }
    // candidate bound of this lane; ceil(x / T) for x <= 4T by comparisons (smax <= 4)
    int T = maxc * (lane + 1) / kWave + 1;
    T = T < 2 * TW ? 2 * TW : T;
    auto nsplit = [&](int x, int t) {
        const int s = 1 + (x > t) + (x > 2 * t) + (x > 3 * t);
        return s < smax ? s : smax;
    };
    const int hpl = Hkv / tmv::kXcds;     // heads per XCD slot
    int need = 0;
    for (int c = 0; c < B; ++c)
        need += hpl * __builtin_amdgcn_readlane(nbl, c) * nsplit(__builtin_amdgcn_readlane(ch, c), T);
    const uint64_t ok = __builtin_amdgcn_ballot_w64(need <= static_cast<int>(gridDim.x / tmv::kXcds));
    const int sel = ok ? __builtin_ctzll(ok) : kWave - 1;
    const int Ts = __builtin_amdgcn_readlane(T, sel);
    // item j of slot x
    const int x = blockIdx.x & (tmv::kXcds - 1), j = blockIdx.x / tmv::kXcds;
    AdaptItem it = {-1, 0, 0, 1, -1};
    int acc = 0;
    for (int c = 0; c < B; ++c) {
        const int n = __builtin_amdgcn_readlane(nbl, c);
        const int s = nsplit(__builtin_amdgcn_readlane(ch, c), Ts);
        const int cnt = hpl * n * s;
        if (j < acc + cnt) {
            const int loc = j - acc, per_head = n * s;
            const int h = loc / per_head, rem = loc - h * per_head;
            it.pair = c * Hkv + x + tmv::kXcds * h;
            it.rbk = rem / s;
            it.split = rem - it.rbk * s;
            it.splits = s;
            // the sequence's last row group (split 0) also clears the rows no item covers
            it.tail_from = (it.rbk == n - 1 && it.split == 0) ? n * RB : -1;
            break;
        }
        acc += cnt;
    }
    return it;
}

template <int D, int RW, bool DEEP, bool PAGED, bool ADAPT>
__global__ void __launch_bounds__(kRingWaves * kWave)
tree_attn_bf16_kernel(const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
                      const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
                      uint32_t ks0_16, uint32_t ks1_16, uint32_t ks2_16, int L_cap, int pairs, uint32_t geom,
                      // (the arguments above fill the 14 SGPRs the hardware preloads: everything
                      // the first K/V copies need, cache strides in 16-byte units; the rest
                      // arrive through the kernel-argument segment)
                      int M_max, int D_max, int nb,
                      const uint16_t *__restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
                      const int32_t *__restrict__ anc, const int32_t *__restrict__ depth,
                      int32_t *__restrict__ status, float qk_scale_log2,
                      uint16_t *__restrict__ out, int64_t os0, int64_t os1, int64_t os2,
                      float *__restrict__ ws_stats, uint16_t *__restrict__ ws_o, uint64_t *__restrict__ ws_cnt,
                      PagedArgs pg)
{
    using RS = RingShape<D>;
    static_assert(D == 128, "the LDS-ring kernel is written for head dimension 128");
    static_assert(RW == 2 || RW == 4 || RW == 8, "row groups of 64, 128 or 256 rows");
    constexpr int KS = D / 32;           // k-steps of the QK^T contraction
    constexpr int NT = D / 16;           // 16-dim output tiles
    constexpr int TW = kRingWaves / RW;  // token groups of waves
    constexpr int RB = RW * kRowsPerWave;
    constexpr int PP = RS::kPieces;
    constexpr int kThreads = kRingWaves * kWave;
    constexpr int kDW = RS::kDmaPerWave;

    // the ring: kNR groups of kR chunk slots, one round of copies each.  A round holds a
    // chunk for every token group (rounds of 2 chunks when the waves form at most 2 token
    // groups, so that up to 3 rounds are in flight while one is computed).  The groups are
    // separate LDS arrays, and the chunk loop names each group it touches statically: the
    // compiler then tells them apart, so a read of one group never waits for the copies
    // still in flight into another (it waits for the group's own copies, which the loop's
    // schedule has already waited for).
    constexpr int kR = TW > 2 ? TW : 2;
    constexpr int kNR = RS::kSlots / kR;
    static_assert(kNR * kR == RS::kSlots && kNR >= 2 && kNR <= 4, "ring groups");
    constexpr int kGroupBytes = kR * RS::kSlotBytes;
    __shared__ __attribute__((aligned(256))) char ring0[kGroupBytes];
    __shared__ __attribute__((aligned(256))) char ring1[kGroupBytes];
    __shared__ __attribute__((aligned(256))) char ring2[kNR > 2 ? kGroupBytes : 16];
    __shared__ __attribute__((aligned(256))) char ring3[kNR > 3 ? kGroupBytes : 16];
    auto group = [&](int gi) -> char * { return gi == 0 ? ring0 : gi == 1 ? ring1 : gi == 2 ? ring2 : ring3; };
    // 64- and 128-row groups read their chunk operands with the inline-assembly blocks (each
    // waits for its own reads) in a rolled loop: the compiler's freedom to hoist ordinary
    // loads, and the unrolled loop they need, cost these kernels more registers than they
    // save time
    constexpr bool kAsmReads = RW <= 4;
    __shared__ float s_ml[kRingWaves * kRowsPerWave * 2];
    // 64-row groups (contiguous caches): the four token groups of a row group share one
    // copy of its query fragments, each loading one k-step (16 KB for the workgroup)
    constexpr bool kShareQ = RW == 2 && TW == KS && !PAGED;
    __shared__ __attribute__((aligned(16))) u32x4_t q_x[kShareQ ? RW * 2 * KS * kWave : 1];
    __shared__ int s_last;
    // paged caches: this sequence's block-table entries (-1: invalid) and, per wave, the
    // first invalid entry it staged
    __shared__ int32_t pg_lds[PAGED ? kMaxPagesLds : 1];
    __shared__ int pg_bad[kRingWaves];

    // ---- decode the workgroup.  grid = (8 * nb, splits, ceil(pairs / 8)) with x = XCD slot +
    // 8 * row block: the linear workgroup id is x + 8 nb (split + splits z), so every
    // workgroup of one (sequence, kv head) pair has the same id mod 8 and the hardware deals
    // them all to the same XCD.  geom = Hkv | g << 16 | S << 21 (S: the splits, or with
    // adaptive items their bound), a preloaded argument, so the first copies of a
    // non-adaptive kernel wait for no kernel-argument load.  ADAPT kernels (ragged batches)
    // run one workgroup per CU, each taking its work item from adaptive_item (the same XCD
    // slot for all items of a pair).
    const int Hkv = static_cast<int>(geom & 0xffffu), g = static_cast<int>((geom >> 16) & 31u);
    const int S = static_cast<int>((geom >> 21) & 31u);
    int rbk, split, splits, pair, smax, tail_from = -1;
    if constexpr (ADAPT) {
        const AdaptItem it = adaptive_item(prefix_len, n_nodes, pairs / Hkv, Hkv, g, RB, TW, M_max, L_cap, S);
        pair = __builtin_amdgcn_readfirstlane(it.pair);
        if (pair < 0) return;
        rbk = __builtin_amdgcn_readfirstlane(it.rbk);
        split = __builtin_amdgcn_readfirstlane(it.split);
        splits = __builtin_amdgcn_readfirstlane(it.splits);
        tail_from = __builtin_amdgcn_readfirstlane(it.tail_from);
        smax = S;
    } else {
        rbk = blockIdx.x >> 3;
        split = blockIdx.y;
        splits = smax = S;
        // (scattered plans, for tests: split s of a pair sits in XCD slot (pair + s) % 8)
        const int shift = (geom >> 26) & 1 ? split : 0;
        pair = blockIdx.z * tmv::kXcds + ((static_cast<int>(blockIdx.x) - shift) & (tmv::kXcds - 1));
        if (pair >= pairs) return;
    }
    const int b = pair / Hkv, kvh = pair - b * Hkv;
    // row r -> node r / g + 1 by a multiply: exact for r < 4096 and g <= 16
    const int g_magic = (65536 + g - 1) / g;
    auto node_of = [&](int r) { return ((r * g_magic) >> 16) + 1; };

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);     // wave-uniform
    const int rw = wave % RW, tw = wave / RW;
    const int c16 = lane & 15, G = lane >> 4;
    const int R = 1 + M_max, W = D_max + 1;
    const int row0_wg = rbk * RB;
    const int row0 = row0_wg + rw * kRowsPerWave;         // first row of this wave

    // ---- K/V copies.  Split s takes the global 32-token chunks s, s + S, s + 2S, ... (local
    // chunk k = global chunk s + k*S), so the chunks of a split are known before the
    // sequence's length is: the first two rounds go out at once, bounded by the cache
    // capacity L_cap (every slot below it is the caller's memory); later rounds stop at the
    // visible length T.  Rows in [T, L_cap) of a speculatively copied chunk are never
    // visible (their mask bits are clear); V rows among them are zeroed in LDS before use
    // (0 * garbage could be NaN), and chunks entirely beyond T are never computed.
    // Local chunk k sits in slot k % kSlots (group (k / kR) % kNR).
    const int ncap = (L_cap + kChunk - 1) / kChunk;
    const int nk_cap = ncap > split ? (ncap - split + splits - 1) / splits : 0;
    int t_lim = L_cap, nk_lim = nk_cap;       // copy bounds: capacity until T is known

    // DMA lane mapping: instruction i of a chunk covers LDS bytes [i*1 KiB, +1 KiB) of the
    // slot; lane l writes 16 bytes at 16*l.  Within K (or V) the LDS holds row t at
    // t*kRowBytes with its 16-byte pieces XOR-swizzled, so the lane that fills LDS piece
    // (t, pp) reads global piece pp ^ swizzle(t) of row t.  Waves 0-3 move K, 4-7 move V.
    // (paged: ks0_16 is the page stride; a chunk's page is added when it is issued)
    const int64_t head_off = ((PAGED ? 0 : static_cast<int64_t>(b) * ks0_16) + static_cast<int64_t>(kvh) * ks1_16) * 16;
    const int64_t page_bytes = static_cast<int64_t>(ks0_16) * 16;
    const char *kbase = reinterpret_cast<const char *>(kc) + head_off;
    const char *vbase = reinterpret_cast<const char *>(vc) + head_off;
    const int64_t row_bytes = static_cast<int64_t>(ks2_16) * 16;
    static_assert((RS::kDmaPerChunk / 2) % kDW == 0, "a wave must stay within K or V");
    const bool wave_v = wave * kDW >= RS::kDmaPerChunk / 2;
    const char *mbase = wave_v ? vbase : kbase;
    uint32_t dma_off[kDW];
    int dma_lds[kDW];
    // 16-token pages: rows 16-31 of a chunk lie on its second page; every DMA instruction
    // covers 4 rows, all on one page (dma_hi), at offsets relative to that page
    bool dma_hi[kDW];
    const bool two_pages = PAGED && pg.shift == 4;
#pragma unroll
    for (int jd = 0; jd < kDW; ++jd) {
        const int i = wave * kDW + jd;                         // instruction within the chunk
        const int ii = wave_v ? i - RS::kDmaPerChunk / 2 : i;
        const int qpos = ii * 64 + lane;                       // 16-byte LDS piece index
        const int t = qpos / PP, pp = qpos % PP;
        // K rows swizzle their 16-byte pieces by t mod 16, V rows by 2t mod 16 (the V^T reads
        // take four consecutive rows at once; see the V^T reads in compute_chunk)
        const int sw = wave_v ? (2 * t) % PP : t % PP;
        // (from the wave-uniform instruction index: instruction ii covers rows 64*ii/PP ..
        // +64/PP - 1, all on one side of row 16, so the page choice stays scalar)
        static_assert((64 / PP) > 0 && 16 % (64 / PP) == 0, "a DMA instruction must not straddle row 16");
        dma_hi[jd] = two_pages && ii * 64 / PP >= 16;
        dma_off[jd] = static_cast<uint32_t>((dma_hi[jd] ? t - 16 : t) * row_bytes + ((pp ^ sw) * 16));
        dma_lds[jd] = (wave_v ? RS::kMatBytes : 0) + ii * 1024;
    }
    // rows of local chunk k to copy (records stop at t_lim, so loads past it write zeros and
    // touch no memory; chunks past nk_lim load nothing)
    auto chunk_recs = [&](int k) __attribute__((always_inline)) {
        const int t0 = (split + k * splits) * kChunk;
        const int recs = (k < nk_lim) ? t_lim - t0 : 0;
        return recs < 0 ? 0 : (recs > kChunk ? kChunk : recs);
    };
    // paged: the staged table entry of local chunk k's first (which = 0) or second page,
    // -1 when the chunk copies no rows there (indices clamped into the staged entries: a
    // chunk with rows has them there)
    auto page_of = [&](int k, int which) __attribute__((always_inline)) {
        const int t0 = (split + k * splits) * kChunk;
        const int recs = chunk_recs(k);
        const int rows = which == 0 ? (two_pages ? (recs < 16 ? recs : 16) : recs) : (two_pages ? recs - 16 : 0);
        const int n_pg = L_cap >> pg.shift;
        const int p = (t0 >> pg.shift) + which;
        return rows > 0 ? pg_lds[p < n_pg - 1 ? p : n_pg - 1] : -1;
    };
    // issue this wave's share of local chunk k into the slot at `slot` (paged: pa / pb are
    // its page entries, wave-uniform)
    auto issue_chunk = [&](int k, char *slot_p, int pa, int pb) __attribute__((always_inline)) {
        const int t0 = (split + k * splits) * kChunk;
        int recs = (k < nk_lim) ? t_lim - t0 : 0;
        recs = recs < 0 ? 0 : (recs > kChunk ? kChunk : recs);
        if constexpr (PAGED) {
            // the chunk's rows on its page(s); an invalid page loads nothing (the sequence
            // is rejected in the prologue when such a page is visible).  (The row count is
            // wave-uniform; readfirstlane keeps the descriptors in scalar registers.)
            const int rs = __builtin_amdgcn_readfirstlane(recs);
            const int recs0 = two_pages ? (rs < 16 ? rs : 16) : rs;
            const int recs1 = two_pages ? (rs > 16 ? rs - 16 : 0) : 0;
            const int64_t in_page = static_cast<int64_t>(t0 & ((1 << pg.shift) - 1)) * row_bytes;
            const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(mbase + (pa >= 0 ? pa : 0) * page_bytes + in_page), 0,
                pa >= 0 ? static_cast<int>(recs0 * row_bytes) : 0, kBufferFlags);
            const __amdgpu_buffer_rsrc_t rbuf = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(mbase + (pb >= 0 ? pb : 0) * page_bytes), 0,
                pb >= 0 ? static_cast<int>(recs1 * row_bytes) : 0, kBufferFlags);
            // (the page choice goes through readfirstlane as an integer: selected as a lane mask,
            // the descriptor would land in vector registers and every copy would become a
            // waterfall loop)
#pragma unroll
            for (int jd = 0; jd < kDW; ++jd)
                dma_to_lds16(__builtin_amdgcn_readfirstlane(dma_hi[jd] ? 1 : 0) ? rbuf : ra, slot_p + dma_lds[jd], dma_off[jd]);
        } else {
            const int nbytes = __builtin_amdgcn_readfirstlane(static_cast<int>(recs * row_bytes));
            const __amdgpu_buffer_rsrc_t mr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<char *>(mbase + static_cast<int64_t>(k < nk_lim ? t0 : 0) * row_bytes), 0, nbytes, kBufferFlags);
#pragma unroll
            for (int jd = 0; jd < kDW; ++jd)
                dma_to_lds16(mr, slot_p + dma_lds[jd], dma_off[jd]);
        }
    };
    // paged: page entries of the next round to issue, read from LDS a round ahead so the
    // read's latency hides behind that round's wait and compute
    int pf_a[kR], pf_b[kR];
    auto prefetch_pages = [&](int r) __attribute__((always_inline)) {
        if constexpr (PAGED) {
#pragma unroll
            for (int j = 0; j < kR; ++j) {
                pf_a[j] = page_of(r * kR + j, 0);
                pf_b[j] = page_of(r * kR + j, 1);
            }
        }
    };
    // round r fills group r % kNR of the ring with local chunks r*kR .. +kR (paged: from
    // the prefetched entries when `prefetched`).  Every wave issues exactly kR * kDW copies
    // per round, empty ones included, so the count of copies issued after a round -- what
    // the waits below rely on -- is the same on every path.
    // (gi: the group, r % kNR -- a constant in the unrolled chunk loop)
    auto issue_round = [&](int gi, int r, bool prefetched = false) __attribute__((always_inline)) {
        char *grp = group(gi);
        if constexpr (PAGED) {
#pragma unroll
            for (int j = 0; j < kR; ++j) {
                const int k = r * kR + j;
                const int pa = __builtin_amdgcn_readfirstlane(prefetched ? pf_a[j] : page_of(k, 0));
                const int pb = __builtin_amdgcn_readfirstlane(prefetched ? pf_b[j] : page_of(k, 1));
                issue_chunk(k, grp + j * RS::kSlotBytes, pa, pb);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kR; ++j) issue_chunk(r * kR + j, grp + j * RS::kSlotBytes, -1, -1);
        }
    };
    // the first kNR rounds, before the chunk loop (every slot of the ring)
    auto issue_prologue = [&](bool from_first) __attribute__((always_inline)) {
        if constexpr (kAsmReads) {
#pragma unroll 1
            for (int r = from_first ? 0 : 1; r < kNR; ++r) issue_round(r, r);
            return;
        }
        if (from_first) issue_round(0, 0);
        issue_round(1, 1);
        if constexpr (kNR > 2) {
            issue_round(2, 2);
            issue_round(3 % kNR, 3);
        }
    };
    // paged caches: this thread's block-table entries are loaded first, together with the
    // prologue's loads below, and staged in LDS before the first copies (L_cap = entries x page)
    constexpr int kPgPer = kMaxPagesLds / kThreads;
    int pg_reg[PAGED ? kPgPer : 1];
    if constexpr (PAGED) {
        const int n_pg = L_cap >> pg.shift;
        const int32_t *trow = pg.tab + static_cast<int64_t>(b) * pg.stride;
#pragma unroll
        for (int u = 0; u < kPgPer; ++u) {
            const int i = threadIdx.x + u * kThreads;
            pg_reg[u] = i < n_pg ? trow[i] : -1;
        }
    } else {
        // the first round goes out before anything else is loaded or waited for
        issue_round(0, 0);
    }

    // ---- the prologue's loads, between the first and the second round of copies (vector
    // loads complete in issue order, so these wait for the first round only): the
    // sequence's scalars and, independently of them, this lane's query fragments, node
    // depths and ancestor entries.  Lane group G fetches entries 4G .. 4G+3 of its rows'
    // ancestor lists; the four groups' mask bits are OR-ed together below.  (Row indices
    // are clamped into the tables, so no load waits on another.)
    const int M = __builtin_amdgcn_readfirstlane(n_nodes[b]);
    const int P = __builtin_amdgcn_readfirstlane(prefix_len[b]);
    int st = __builtin_amdgcn_readfirstlane(status[b]);
    bf16x8_t qf[2][KS];
    int dep[2], ancq[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        int r = row0 + rt * 16 + c16;
        if (r > M_max * g - 1) r = M_max * g - 1;
        const int j = node_of(r), gi = r - (j - 1) * g;
        const uint16_t *qp = q + b * qs0 + static_cast<int64_t>(j - 1) * qs1 + static_cast<int64_t>(kvh * g + gi) * qs2 + G * 8;
        // (with a shared query tile each token group loads one k-step: see below)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            if (!kShareQ || ks == tw) qf[rt][ks] = load_bf16x8(qp + ks * 32);
        dep[rt] = depth[static_cast<int64_t>(b) * R + j];
        const int32_t *arow = anc + (static_cast<int64_t>(b) * R + j) * W;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int kk = 4 * G + k;
            ancq[rt][k] = arow[kk < W ? kk : W - 1];
        }
    }
    if constexpr (!PAGED) issue_prologue(false);
    if constexpr (PAGED) {
        // stage the entries (invalid ones as -1; each wave records the first invalid one),
        // then issue the first two rounds from them
        const int n_pg = L_cap >> pg.shift;
        int bad_min = 0x7fffffff;
#pragma unroll
        for (int u = 0; u < kPgPer; ++u) {
            const int i = threadIdx.x + u * kThreads;
            if (i < n_pg) {
                const int e = pg_reg[u];
                const bool ok = e >= 0 && e < pg.npages;
                pg_lds[i] = ok ? e : -1;
                bad_min = ok || i > bad_min ? bad_min : i;
            }
        }
        for (int o = 32; o >= 1; o >>= 1) {
            const int y = __shfl_xor(bad_min, o, kWave);
            bad_min = y < bad_min ? y : bad_min;
        }
        if (lane == 0) pg_bad[wave] = bad_min;
        __syncthreads();
        issue_prologue(true);
    }

    if (st == TMV_OK && (M < 0 || M > M_max || P < 0 || static_cast<int64_t>(P) + M > L_cap)) {
        st = TMV_ERR_INPUT;
        if (threadIdx.x == 0 && rbk == 0 && split == 0) status[b] = TMV_ERR_INPUT;
    }
    if constexpr (PAGED) {
        // every page holding a visible token must be a valid page
        int fb = pg_bad[0];
#pragma unroll
        for (int w = 1; w < kRingWaves; ++w) fb = pg_bad[w] < fb ? pg_bad[w] : fb;
        fb = __builtin_amdgcn_readfirstlane(fb);
        if (st == TMV_OK && fb < ((P + M + (1 << pg.shift) - 1) >> pg.shift)) {
            st = TMV_ERR_INPUT;
            if (threadIdx.x == 0 && rbk == 0 && split == 0) status[b] = TMV_ERR_INPUT;
        }
    }
    const int Rh = (st == TMV_OK) ? M * g : 0;           // live rows of this kv head

    // adaptive items: the last row group of a sequence also clears its output rows from
    // tail_from on, which no item covers (zeros, as for any inert row)
    auto clear_tail = [&]() {
        if (tail_from < 0) return;
        const int rows = M_max * g - tail_from;
        for (int i = threadIdx.x; i < rows * (D / 8); i += kThreads) {
            const int r = tail_from + i / (D / 8), e = (i % (D / 8)) * 8;
            const int j = node_of(r), gi = r - (j - 1) * g;
            *reinterpret_cast<uint4 *>(out + b * os0 + static_cast<int64_t>(j - 1) * os1 +
                                       static_cast<int64_t>(kvh * g + gi) * os2 + e) = make_uint4(0, 0, 0, 0);
        }
    };
    if (row0_wg >= Rh) {
        clear_tail();
        // no live row in this workgroup (nor in the other splits of its row block, which
        // see the same rows): split 0 clears the block's output rows
        if (split == 0 && tw == 0) {
            for (int rt = 0; rt < 2; ++rt) {
                const int r = row0 + rt * 16 + c16;
                if (r >= M_max * g) continue;
                const int j = node_of(r), gi = r - (j - 1) * g;
                uint16_t *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + static_cast<int64_t>(kvh * g + gi) * os2 + G * (D / 4);
#pragma unroll
                for (int e = 0; e < D / 4; e += 8) *reinterpret_cast<uint4 *>(o + e) = make_uint4(0, 0, 0, 0);
            }
        }
        __builtin_amdgcn_s_waitcnt(kVmcntZero);   // no copy may land in LDS after the exit
        return;
    }

    // ---- this split's chunks of the visible range [0, T); later copies stop at T
    const int T = P + M;                                  // tokens visible to someone
    const int nchunks = (T + kChunk - 1) / kChunk;
    const int nk = __builtin_amdgcn_readfirstlane(nchunks > split ? (nchunks - split + splits - 1) / splits : 0);
    const int nrounds = (nk + kR - 1) / kR;
    t_lim = T;
    nk_lim = nk;
    // the chunk holding T when T is not a chunk boundary: its rows >= T may hold anything
    // if it was copied before T was known (the first kNR rounds of the first pass)
    const int cb = T / kChunk;
    const int kb_loc = (T % kChunk != 0 && cb >= split && (cb - split) % splits == 0) ? (cb - split) / splits : -1;
    const int kb_round = kb_loc >= 0 && kb_loc < RS::kSlots ? kb_loc / kR : -1;

    const bool wave_live = row0 < Rh;

    // ---- ancestor-or-self masks of the lane's two rows as four 32-bit words (bit a of the
    // mask <-> tree slot P + a); rows beyond the live ones are padding whose results are
    // never written.  A bit index outside [0, 128) sets nothing.
    uint32_t mw[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int w = 0; w < 4; ++w) mw[rt][w] = 0u;
        const int r = row0 + rt * 16 + c16;
        if (r >= Rh) continue;
        const int dp = dep[rt];
        auto set_bit = [&](int a) {
#pragma unroll
            for (int w = 0; w < 4; ++w) mw[rt][w] |= (a >> 5) == w ? (1u << (a & 31)) : 0u;
        };
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (4 * G + k < dp) set_bit(ancq[rt][k] - 1);
        if (DEEP && dp > kAncBatch) {
            // deep rows: the rest of the path, one batch of loads per round trip
            const int j = node_of(r);
            const int32_t *arow = anc + (static_cast<int64_t>(b) * R + j) * W;
            for (int k0 = kAncBatch; k0 < dp; k0 += kAncBatch) {
                int e[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int kk = k0 + 4 * G + k;
                    e[k] = arow[kk < W ? kk : W - 1];
                }
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (k0 + 4 * G + k < dp) set_bit(e[k] - 1);
            }
        }
    }
    // OR the four lane groups' bits (lanes c16, c16 + 16, c16 + 32, c16 + 48 hold one row)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const auto x16 = __builtin_amdgcn_permlane16_swap(mw[rt][w], mw[rt][w], false, false);
            const uint32_t y = x16[0] | x16[1];
            const auto x32 = __builtin_amdgcn_permlane32_swap(y, y, false, false);
            mw[rt][w] = x32[0] | x32[1];
        }

    // the query fragments carry the score scale (scale * log2 e, rounded to bf16 once), so
    // the score MFMAs yield base-2 exponents directly (with a shared query tile each wave
    // scales the k-step it loaded)
    auto scale_q = [&](bf16x8_t x) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = static_cast<__bf16>(static_cast<float>(x[e]) * qk_scale_log2);
        return x;
    };
    if constexpr (kShareQ) {
        // exchange the query k-steps: write this wave's, barrier, read all (LDS operations
        // in inline assembly: a compiler-written one would first wait for every copy in flight)
        const uint32_t qb = lds_addr(reinterpret_cast<const char *>(q_x));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                if (ks == tw) lds_write16(qb + (((rw * 2 + rt) * KS + ks) * kWave + lane) * 16, __builtin_bit_cast(u32x4_t, scale_q(qf[rt][ks])));
        __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
        __builtin_amdgcn_s_barrier();
        uint32_t qa[2 * KS];
        u32x4_t qv[2 * KS];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[rt * KS + ks] = qb + (((rw * 2 + rt) * KS + ks) * kWave + lane) * 16;
        lds_read_b128_x8(qv, qa);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = __builtin_bit_cast(bf16x8_t, qv[rt * KS + ks]);
    }

    if constexpr (!kShareQ) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = scale_q(qf[rt][ks]);
    }
    // LDS read offsets of the MFMA operands inside a slot (constant per lane).  K
    // fragment (tt, ks): row tt*16 + c16, logical piece ks*4 + G.  V^T: lane reads row
    // h*16 + 4G + c16/4 at dims 4*(c16%4) of each 16-dim tile (offset zv[h]; see compute_chunk).
    uint32_t lk[2][KS], zv[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int t = tt * 16 + c16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) lk[tt][ks] = t * RS::kRowBytes + (((ks * 4 + G) ^ (t % PP)) * 16);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int t = h * 16 + 4 * G + (c16 >> 2);
        zv[h] = RS::kMatBytes + t * RS::kRowBytes + (((c16 & 3) >> 1) * 16) + (c16 & 1) * 8 + ((2 * t) % PP) * 16;
    }

    f32x4_t oacc[2][NT];
    // row sums of p come out of the PV product itself: an extra dim tile whose A operand is
    // 1 at tile dim 0 and 0 elsewhere accumulates, at dim 0, the sum of the bf16 p of each
    // row (exactly the weights the rows of O receive); lane (c16, G = 0) holds row c16's sum
    f32x4_t lacc[2];
    const uint32_t one2 = c16 == 0 ? 0x3F803F80u : 0u;                 // two bf16 ones
    const bf16x8_t ones_a = __builtin_bit_cast(bf16x8_t, make_uint4(one2, one2, one2, one2));
    float mref[2], mlane[2], lrow[2];
    // minit[rt]: the score MFMAs' initial accumulator, minus the row's reference (0 while it
    // is unset), so that they yield each score's exponent relative to the reference
    f32x4_t minit[2];
    // maxima of scores in IEEE maximum form (a NaN score propagates; -0 and +0 need no
    // care here): unlike fmaxf it needs no quieting of MFMA results first
    auto vmax = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
    auto xor16_max = [&](float x) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    auto xor32_max = [&](float x) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
    };
    // first pass: each row's reference is the first finite chunk maximum (O and l are
    // still exactly zero then, so adopting it rescales nothing); later maxima are only
    // tracked, per lane, relative to the reference (a row's maximum is the maximum over its
    // four lanes, taken only when needed).  p = 2^(score exponent - ref) stays finite
    // unless an exponent exceeds the reference by more than kOverflow, in which case the
    // whole split is recomputed against the exact maximum -- the accumulators never need
    // rescaling inside the loop.
    bool first_pass = true;
    // every row of the wave has its reference (wave-uniform; first pass only)
    bool ref_ready = false;
    // softmax weights of a chunk's scores (cm: this lane's maxima of them) and the PV product
    auto lane_max = [&](const f32x4_t (&s)[2]) {
        return vmax(vmax(vmax(s[0][0], s[0][1]), vmax(s[0][2], s[0][3])),
                    vmax(vmax(s[1][0], s[1][1]), vmax(s[1][2], s[1][3])));
    };
    auto finish_chunk = [&](f32x4_t (&s)[2][2], const u32x2_t (&vt)[16], float (&cm)[2]) {
        if (first_pass && !ref_ready) {
            // a row without a reference takes this chunk's row maximum (scores of such a row
            // are absolute; they become relative here)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                if (__builtin_amdgcn_ballot_w64(mref[rt] == -INFINITY) == 0) continue;
                const float rm = xor32_max(xor16_max(cm[rt]));
                if (mref[rt] == -INFINITY && rm != -INFINITY) {
                    mref[rt] = rm;
                    cm[rt] -= rm;
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i) s[rt][tt][i] -= rm;
                    minit[rt] = f32x4_t{-rm, -rm, -rm, -rm};
                }
            }
            ref_ready = __builtin_amdgcn_ballot_w64(mref[0] == -INFINITY || mref[1] == -INFINITY) == 0;
        }
        // each lane's largest exponent relative to its row's reference (a row whose reference
        // is still unset has no finite score in this lane)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) mlane[rt] = vmax(mlane[rt], cm[rt]);
        bf16x8_t pb[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) pb[rt][tt * 4 + i] = static_cast<__bf16>(__builtin_amdgcn_exp2f(s[rt][tt][i]));
        // O^T += V^T P^T over dim tiles of 16: A operand of tile nt = (tokens pi(8G + j)) at
        // dim nt*16 + c16; the accumulator lane holds dims nt*16 + 4G + i of row c16
        mfma_priority(1);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(vt[2 * nt].x, vt[2 * nt].y, vt[2 * nt + 1].x, vt[2 * nt + 1].y));
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                oacc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], oacc[rt][nt], 0, 0, 0);
        }
        mfma_priority(0);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) lacc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones_a, pb[rt], lacc[rt], 0, 0, 0);
    };
    auto compute_chunk = [&](const char *slot, int c) {
        const int t0 = c * kChunk;
        // S^T tiles: [token][row]; lane holds row c16 of tile rt, tokens t0 + tt*16 + G*4 + i
        constexpr int NK = 2 * KS;                   // K fragments of the chunk per lane
        u32x4_t kraw[NK];
        {
            uint32_t ka[NK];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) ka[tt * KS + ks] = lk[tt][ks];
            if constexpr (kAsmReads) {
                const uint32_t sp = lds_addr(slot);
#pragma unroll
                for (int i = 0; i < NK; ++i) ka[i] += sp;
                lds_read_b128_x8(kraw, ka);
            } else {
#pragma unroll
                for (int i = 0; i < NK; ++i) kraw[i] = *reinterpret_cast<const u32x4_t *>(slot + ka[i]);
            }
        }
        bf16x8_t kf[2][KS];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kf[tt][ks] = __builtin_bit_cast(bf16x8_t, kraw[tt * KS + ks]);
        f32x4_t s[2][2];
        mfma_priority(1);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x4_t acc = minit[rt];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[tt][ks], qf[rt][ks], acc, 0, 0, 0);
                s[rt][tt] = acc;
            }
        mfma_priority(0);
        // this lane's score maxima (a chunk reaching the tree slots takes them again over
        // its visible scores below)
        float cm[2] = {lane_max(s[0]), lane_max(s[1])};
        // V^T fragments go out while the score MFMAs run
        u32x2_t vt[16];
        // V^T operand reads with the gfx950 transposing LDS load: within each 16-lane group,
        // lane s supplies 4 consecutive bf16 at its address and receives element s%4 of the
        // groups supplied by lanes s/4, s/4 + 4, s/4 + 8, s/4 + 12.  With lane s reading row
        // T[s/4] at dims 4*(s%4) .. +3 of a 16-dim tile, lane s ends up with dim s of rows
        // T[0..3] -- one column of V, as the MFMA A operand wants.  vt[2*nt + h]: dim tile
        // nt, token half h; the tile's offset is the lane's half offset zv[h] with 32*nt
        // XORed in (the swizzle of the V rows only permutes 32-byte dim groups).
        if constexpr (kAsmReads) {
            // (the XOR touches bits 5-7 only: a slot starts at a multiple of 256 bytes)
            lds_read_vt(vt, lds_addr(slot) + zv[0], lds_addr(slot) + zv[1]);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                vt[i] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) s16x4_t *)(slot + (zv[i & 1] ^ (32u * (i >> 1))))));
        }
        if (t0 + kChunk > P) {
            // chunk reaches the tree slots: a token is visible if it is in the prefix or is
            // an ancestor-or-self of the row's node.  Over the sequence of 32-bit words
            // (all ones, mask bits 0-31, 32-63, 64-95, 96-127) -- i.e. prefix tokens read as
            // visible -- the chunk's 32 visibility bits start at bit e = t0 - P + 32 (>= 1).
            const int e = t0 - P + 32;
            const int qw = e >> 5, sh = e & 31;                       // wave-uniform
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const uint32_t w0 = mw[rt][0], w1 = mw[rt][1], w2 = mw[rt][2], w3 = mw[rt][3];
                const uint32_t lo = qw == 0 ? 0xFFFFFFFFu : qw == 1 ? w0 : qw == 2 ? w1 : qw == 3 ? w2 : w3;
                const uint32_t hi = qw == 0 ? w0 : qw == 1 ? w1 : qw == 2 ? w2 : qw == 3 ? w3 : 0u;
                const uint32_t win = __builtin_amdgcn_alignbit(hi, lo, sh) >> (G * 4);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s[rt][tt][i] = ((win >> (tt * 16 + i)) & 1u) ? s[rt][tt][i] : -INFINITY;
                cm[rt] = lane_max(s[rt]);
            }
        }
        finish_chunk(s, vt, cm);
    };

#pragma unroll
    for (int rt = 0; rt < 2; ++rt) { mref[rt] = -INFINITY; mlane[rt] = -INFINITY; minit[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; }
    // (the pass, round and slot loops stay rolled: one copy of the chunk code keeps the
    // kernel small enough for the instruction cache)
#pragma unroll 1
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            lacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) oacc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
        if (pass > 0) issue_prologue(true);
        // Round r (ring group r % kNR): wait until this wave's copies of round r have landed
        // (later rounds may still be in flight: vector-memory operations complete in issue
        // order and every wave issues exactly kR * kDW copies per round), barrier -- every
        // wave's share of round r is then visible and every wave has finished reading round
        // r - 1 -- then refill round r - 1's group with round r + kNR - 1 and compute round r.
        // (tmv_ring defines and checks the schedule.)  The barriers carry no memory fence on
        // purpose: a fence would wait for all copies in flight.  The loop is unrolled over
        // the groups so that each group is named statically.
        auto round_body = [&](auto G, int r, auto refill) __attribute__((always_inline)) {
            constexpr int gi = decltype(G)::value;
            char *grp = group(gi);
            if (r == 0) __builtin_amdgcn_s_waitcnt(kVmcntRound<(kNR - 1) * kR * kDW>());
            else __builtin_amdgcn_s_waitcnt(kVmcntRound<(kNR - 2) * kR * kDW>());
            __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
            __builtin_amdgcn_s_barrier();
            if (pass == 0 && r == kb_round) {
                // the chunk holding T was copied before T was known: zero its V rows >= T
                const int r0 = T - (split + kb_loc * splits) * kChunk;
                const uint32_t vb = lds_addr(grp) + (kb_loc % kR) * RS::kSlotBytes + RS::kMatBytes + r0 * RS::kRowBytes;
                for (int i = threadIdx.x; i < (kChunk - r0) * PP; i += kThreads) lds_zero16(vb + i * 16);
                __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
                __builtin_amdgcn_s_barrier();
            }
            if constexpr (decltype(refill)::value) issue_round((gi + kNR - 1) % kNR, r + kNR - 1, true);
            // (paged: the next refill's table entries, read from LDS a round ahead)
            prefetch_pages(r + kNR);
            if (wave_live) {
#pragma unroll 1
                for (int j = tw; j < kR; j += TW) {
                    const int k = r * kR + j;
                    if (k < nk) compute_chunk(grp + j * RS::kSlotBytes, split + k * splits);
                }
            }
        };
        static_assert(tmv_ring::inflight(0, kNR) == kNR - 1 && tmv_ring::inflight(1, kNR) == kNR - 2 &&
                      tmv_ring::issue_at(1, kNR) == kNR, "the loop below follows tmv_ring");
        if constexpr (kAsmReads) {
            // (operands read by the inline-assembly blocks: one copy of the loop, the group
            // chosen at run time, keeps these kernels small.  With two groups every wait is
            // for all copies in flight, so rounds past the last need not be issued.)
#pragma unroll 1
            for (int r = 0; r < nrounds; ++r) {
                char *grp = group(r % kNR);
                if (r == 0) __builtin_amdgcn_s_waitcnt(kVmcntRound<(kNR - 1) * kR * kDW>());
                else __builtin_amdgcn_s_waitcnt(kVmcntRound<(kNR - 2) * kR * kDW>());
                __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
                __builtin_amdgcn_s_barrier();
                if (pass == 0 && r == kb_round) {
                    const int r0 = T - (split + kb_loc * splits) * kChunk;
                    const uint32_t vb = lds_addr(grp) + (kb_loc % kR) * RS::kSlotBytes + RS::kMatBytes + r0 * RS::kRowBytes;
                    for (int i = threadIdx.x; i < (kChunk - r0) * PP; i += kThreads) lds_zero16(vb + i * 16);
                    __builtin_amdgcn_s_waitcnt(kLgkmcntZero);
                    __builtin_amdgcn_s_barrier();
                }
                if (r >= 1 && (kNR > 2 || r + kNR - 1 < nrounds)) issue_round((r + kNR - 1) % kNR, r + kNR - 1, true);
                prefetch_pages(r + kNR);
                if (wave_live) {
#pragma unroll 1
                    for (int j = tw; j < kR; j += TW) {
                        const int k = r * kR + j;
                        if (k < nk) compute_chunk(grp + j * RS::kSlotBytes, split + k * splits);
                    }
                }
            }
        } else {
        if (nrounds > 0) round_body(tmv::Const<0>{}, 0, tmv::Const<0>{});
#pragma unroll 1
        for (int r0 = 1; r0 < nrounds; r0 += kNR) {
            round_body(tmv::Const<1>{}, r0, tmv::Const<1>{});
            if (r0 + 1 >= nrounds) break;
            if constexpr (kNR > 2) {
                round_body(tmv::Const<2 % kNR>{}, r0 + 1, tmv::Const<1>{});
                if (r0 + 2 >= nrounds) break;
                round_body(tmv::Const<3 % kNR>{}, r0 + 2, tmv::Const<1>{});
                if (r0 + 3 >= nrounds) break;
            }
            round_body(tmv::Const<0>{}, r0 + kNR - 1, tmv::Const<1>{});
        }
        }
        __builtin_amdgcn_s_waitcnt(kVmcntZero);   // nothing may land in LDS after this
        // the decision is the workgroup's: every wave must take the same number of passes,
        // since the passes contain barriers
        const bool overflow = first_pass && (mlane[0] > kOverflow || mlane[1] > kOverflow);
        if (!__syncthreads_or(overflow ? 1 : 0)) break;
        // rare: some score outgrew its reference; redo the split against the exact maxima
        first_pass = false;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const float mx = xor32_max(xor16_max(mlane[rt]));
            if (mref[rt] != -INFINITY) mref[rt] += mx;
            minit[rt] = mref[rt] == -INFINITY ? f32x4_t{0.f, 0.f, 0.f, 0.f}
                                              : f32x4_t{-mref[rt], -mref[rt], -mref[rt], -mref[rt]};
        }
    }
    // (the pass loop is only left through the block-wide __syncthreads_or above: every wave
    // has finished reading the ring, so no further barrier is needed before it is reused)
    clear_tail();
    float mrow[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        lrow[rt] = lacc[rt][0];       // the ones tile: lanes with G > 0 hold exact zeros
        // row sums: each of the four lanes of a row holds a partial sum
        auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(lrow[rt]), __float_as_uint(lrow[rt]), false, false);
        const float l16 = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
        auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l16), __float_as_uint(l16), false, false);
        lrow[rt] = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
        // from here on the running maxima are in base-2 units, as the merge steps expect
        mrow[rt] = mref[rt];
    }

    // ---- split-KV completion: the last split of a row block to arrive merges the block.
    // Every workgroup of a row block has the same id mod 8, and the hardware deals a launch's
    // workgroups round-robin to the 8 XCDs, so the block's splits share one XCD and its L2:
    // they publish their partials with plain stores (the L1s write through to that L2) and
    // the merging workgroup reads them from the L2 -- the partials need not travel to memory
    // and back.  A split's stores are complete once its vector-memory count drains, after
    // which it counts itself in with a device-scope atomic on the block's 64-bit arrival
    // word, adding 1 to the 8-bit count of its own XCD (HW_REG_XCC_ID).  The last arrival
    // clears the word; if every other arrival came from its XCD it merges, otherwise (a
    // dispatch that split the block over several XCDs, whose L2s do not see each other's
    // stores) it writes the block's rows as zeros and marks the sequence TMV_ERR_DEVICE.
    // this launch's split partials: [pairs * nb units][smax][RB rows] (m, l) and O rows
    const int64_t part_rows = static_cast<int64_t>(pairs) * nb * smax * RB;
    const __amdgpu_buffer_rsrc_t part_o =
        __builtin_amdgcn_make_buffer_rsrc(ws_o, 0, static_cast<int>(part_rows * D * 2), kBufferFlags);
    const __amdgpu_buffer_rsrc_t part_ml =
        __builtin_amdgcn_make_buffer_rsrc(ws_stats, 0, static_cast<int>(part_rows * 8), kBufferFlags);
    const int64_t unit = static_cast<int64_t>(pair) * nb + rbk;
    auto finish_split = [&]() {
        __builtin_amdgcn_s_waitcnt(kVmcntZero);
        __syncthreads();
        if (threadIdx.x == 0) {
            unsigned xcc;
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
            const int sh = 8 * static_cast<int>(xcc & 7u);
            const uint64_t old = __hip_atomic_fetch_add(ws_cnt + unit, uint64_t(1) << sh, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
            int arrived = 0;
#pragma unroll
            for (int x = 0; x < tmv::kXcds; ++x) arrived += static_cast<int>((old >> (8 * x)) & 0xffu);
            s_last = arrived != splits - 1 ? 0 : old == (static_cast<uint64_t>(splits - 1) << sh) ? 1 : 2;
        }
        __syncthreads();
        if (s_last == 0) return;
        int mst = st;
        if (threadIdx.x == 0) {
            __hip_atomic_store(ws_cnt + unit, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (s_last == 2 && st == TMV_OK) status[b] = TMV_ERR_DEVICE;
        }
        if (s_last == 2) mst = TMV_ERR_DEVICE;       // the block's rows are written as zeros
        // (the ring is idle: the merge stages the statistics in its first group)
        if (splits <= 8)
            merge_block<D, RB, 8>(unit, splits, smax, b, kvh, g, g_magic, row0_wg, M_max, L_cap, M, P, mst, depth, out,
                                  os0, os1, os2, ws_stats, ws_o, reinterpret_cast<float *>(ring0));
        else
            merge_block<D, RB, 16>(unit, splits, smax, b, kvh, g, g_magic, row0_wg, M_max, L_cap, M, P, mst, depth, out,
                                   os0, os1, os2, ws_stats, ws_o, reinterpret_cast<float *>(ring0));
    };
    // row `rr` of the workgroup's block, dims d0 .. d0 + n - 1 (n a multiple of 8) of the
    // final output (splits == 1) from x / l, or zeros for inert rows
    auto write_row = [&](int rr, int d0, const float *x, int n, float l) {
        const int r = row0_wg + rr;
        if (r >= M_max * g) return;
        const int j = node_of(r), gi = r - (j - 1) * g;
        const bool live = r < Rh && depth[static_cast<int64_t>(b) * R + j] >= 1;
        const float inv = live && l > 0.f ? 1.f / l : 0.f;
        uint16_t *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + static_cast<int64_t>(kvh * g + gi) * os2 + d0;
        for (int e = 0; e < n; e += 8) {
            uint32_t w4[4];
#pragma unroll
            for (int h2 = 0; h2 < 4; ++h2) {
                const float x0 = live ? x[e + 2 * h2] * inv : 0.f, x1 = live ? x[e + 2 * h2 + 1] * inv : 0.f;
                w4[h2] = tmv::pack_bf16x2(x0, x1);
            }
            *reinterpret_cast<uint4 *>(o + e) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
    };

    if constexpr (TW > 1) {
        // ---- the TW token groups share each row group: every wave parks its (m, l, O) in
        // the idle ring (16 KB per wave; 4-float groups XOR-swizzled by row so the parked
        // writes are free of bank conflicts), then each wave combines its share of its row
        // group's rows over the group's TW waves in a fixed order.
        constexpr int kParkBytes = kRowsPerWave * D * 4;
        static_assert(kRingWaves * kParkBytes == kNR * kGroupBytes && kGroupBytes % kParkBytes == 0, "park area = ring");
        auto parked = [&](int w) {
            constexpr int per = kGroupBytes / kParkBytes;
            return reinterpret_cast<float *>(group(w / per) + (w % per) * kParkBytes);
        };
        {
            float *o = parked(wave);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int rr = rt * 16 + c16;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    *reinterpret_cast<f32x4_t *>(o + rr * D + (((nt * 4 + G) ^ (rr & 31)) << 2)) = oacc[rt][nt];
                if (G == 0) *reinterpret_cast<float2 *>(s_ml + (wave * kRowsPerWave + rr) * 2) = make_float2(mrow[rt], lrow[rt]);
            }
        }
        __syncthreads();
        // wave (rw, tw) combines rows tw*RPW .. +RPW of row group rw; LPR lanes per row,
        // DL dims per lane
        constexpr int RPW = kRowsPerWave / TW, LPR = kWave / RPW, DL = D / LPR;
        const int rg = tw * RPW + lane / LPR, d0 = (lane % LPR) * DL;
        const int rr = rw * kRowsPerWave + rg;                      // row within the workgroup
        float mw_[TW], lw_[TW], mt = -INFINITY;
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const float2 x = *reinterpret_cast<const float2 *>(s_ml + ((w * RW + rw) * kRowsPerWave + rg) * 2);
            mw_[w] = x.x; lw_[w] = x.y;
            mt = fmaxf(mt, x.x);
        }
        const float mref2 = mt == -INFINITY ? 0.f : mt;
        float sc[TW], lt = 0.f;
#pragma unroll
        for (int w = 0; w < TW; ++w) { sc[w] = __builtin_amdgcn_exp2f(mw_[w] - mref2); lt += sc[w] * lw_[w]; }
        float acc[DL];
#pragma unroll
        for (int e = 0; e < DL; ++e) acc[e] = 0.f;
#pragma unroll
        for (int w = 0; w < TW; ++w) {
            const float *src = parked(w * RW + rw) + rg * D;
#pragma unroll
            for (int e = 0; e < DL; e += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(src + ((((d0 + e) >> 2) ^ (rg & 31)) << 2));
                acc[e] += sc[w] * x.x; acc[e + 1] += sc[w] * x.y; acc[e + 2] += sc[w] * x.z; acc[e + 3] += sc[w] * x.w;
            }
        }
        if (splits > 1) {
            // ---- publish this split's partial: (m, l) and the row normalised by l in bf16
            const int base = static_cast<int>((unit * smax + split) * RB);
            const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
            for (int e = 0; e < DL; e += 8) {
                u32x4_t x;
#pragma unroll
                for (int h2 = 0; h2 < 4; ++h2)
                    x[h2] = tmv::pack_bf16x2(acc[e + 2 * h2] * inv, acc[e + 2 * h2 + 1] * inv);
                __builtin_amdgcn_raw_buffer_store_b128(x, part_o, ((base + rr) * D + d0 + e) * 2, 0, 0);
            }
            if ((lane % LPR) == 0) {
                const u32x2_t x = {__float_as_uint(mt), __float_as_uint(lt)};
                __builtin_amdgcn_raw_buffer_store_b64(x, part_ml, (base + rr) * 8, 0, 0);
            }
            finish_split();
            return;
        }
        write_row(rr, d0, acc, DL, lt);
    } else {
        // ---- one token group: every wave holds whole rows (lane: dims nt*16 + 4G .. +3)
        if (splits > 1) {
            const int base = static_cast<int>((unit * smax + split) * RB + rw * kRowsPerWave);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int rr = rt * 16 + c16;
                const float inv = lrow[rt] > 0.f ? 1.f / lrow[rt] : 0.f;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const u32x2_t x = {tmv::pack_bf16x2(oacc[rt][nt][0] * inv, oacc[rt][nt][1] * inv),
                                       tmv::pack_bf16x2(oacc[rt][nt][2] * inv, oacc[rt][nt][3] * inv)};
                    __builtin_amdgcn_raw_buffer_store_b64(x, part_o, ((base + rr) * D + nt * 16 + 4 * G) * 2, 0, 0);
                }
                if (G == 0) {
                    const u32x2_t x = {__float_as_uint(mrow[rt]), __float_as_uint(lrow[rt])};
                    __builtin_amdgcn_raw_buffer_store_b64(x, part_ml, (base + rr) * 8, 0, 0);
                }
            }
            finish_split();
            return;
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int r = row0 + rt * 16 + c16;
            if (r >= M_max * g) continue;
            const int j = node_of(r), gi = r - (j - 1) * g;
            const bool live = r < Rh && depth[static_cast<int64_t>(b) * R + j] >= 1;
            const float inv = live && lrow[rt] > 0.f ? 1.f / lrow[rt] : 0.f;
            uint16_t *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + static_cast<int64_t>(kvh * g + gi) * os2 + 4 * G;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float x0 = live ? oacc[rt][nt][0] * inv : 0.f, x1 = live ? oacc[rt][nt][1] * inv : 0.f;
                const float x2 = live ? oacc[rt][nt][2] * inv : 0.f, x3 = live ? oacc[rt][nt][3] * inv : 0.f;
                *reinterpret_cast<uint2 *>(o + nt * 16) = make_uint2(tmv::pack_bf16x2(x0, x1), tmv::pack_bf16x2(x2, x3));
            }
        }
    }
}

// --------------------------------------------------------------------------- fp32 kernel
// One workgroup of 4 waves per (sequence, node, query head); wave w takes the 64-token
// chunks w, w + 4, w + 8, ... of the row's visible tokens (prefix, then its path), so a
// short row's chunks are all in flight at once instead of one after another.  Within a
// chunk each lane scores one token: its K row arrives as D/4 independent 16-byte loads
// against the query held in registers.  The chunk's V rows go out together with the K
// rows, each one coalesced row at a wave-uniform address (readlane of the token's slot),
// lanes holding dims lane and lane + 64; prefix tokens need no ancestor-table read, so a
// prefix chunk's loads leave as soon as the prefix length is known.  Each wave keeps a
// running (max, sum, weighted V) and the four are combined in LDS at the end.
template <int D>
__global__ void __launch_bounds__(256)
tree_attn_f32_kernel(int B, int M_max, int D_max, int Hq, int Hkv,
                     const float *__restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
                     const float *__restrict__ kc, const float *__restrict__ vc,
                     int64_t ks0, int64_t ks1, int64_t ks2, int L_cap,
                     const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
                     const int32_t *__restrict__ anc, const int32_t *__restrict__ depth,
                     int32_t *__restrict__ status, float scale,
                     float *__restrict__ out, int64_t os0, int64_t os1, int64_t os2)
{
    constexpr int DV = D / 64;                 // output dims per lane
    constexpr int kBatch = 64 / DV;            // V rows per batch (a chunk is 64 tokens)
    constexpr int kFw = 4;                     // waves per row
    __shared__ float red_ml[kFw][2];
    __shared__ float red_acc[kFw][D];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t item = blockIdx.x;
    const int h = static_cast<int>(item % Hq);
    const int j = static_cast<int>((item / Hq) % M_max) + 1;
    const int b = static_cast<int>(item / (static_cast<int64_t>(Hq) * M_max));
    const int g = Hq / Hkv, kvh = h / g;
    const int R = M_max + 1, W = D_max + 1;
    float *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + h * os2;

    // every load that does not depend on another goes out at once: the sequence's counts,
    // the node's depth, its ancestor row (lane k holds entries k, 64 + k, 128 + k) and its
    // query row -- all inside their tables whatever they hold -- so the launch waits for one
    // round trip before the K/V loads instead of one per dependent step
    const int32_t *arow = anc + (static_cast<int64_t>(b) * R + j) * W;
    const int M = n_nodes[b], P = prefix_len[b];
    int st = status[b];
    const int dep_in = depth[static_cast<int64_t>(b) * R + j];
    int a3[3];
#pragma unroll
    for (int k = 0; k < 3; ++k) a3[k] = arow[min(64 * k + lane, W - 1)];
    const float *qp = q + b * qs0 + static_cast<int64_t>(j - 1) * qs1 + h * qs2;
    float4 qv[D / 4];
#pragma unroll
    for (int e = 0; e < D / 4; ++e) qv[e] = reinterpret_cast<const float4 *>(qp)[e];
    if (st == TMV_OK && (M < 0 || M > M_max || P < 0 || static_cast<int64_t>(P) + M > L_cap)) {
        st = TMV_ERR_INPUT;
        if (threadIdx.x == 0 && j == 1 && h == 0) status[b] = TMV_ERR_INPUT;
    }
    const int dep = (st == TMV_OK && j <= M) ? dep_in : 0;
    if (dep < 1) {
        if (wv == 0)
#pragma unroll
            for (int e = 0; e < DV; ++e) o[lane + 64 * e] = 0.f;
        return;
    }

    const float *kb = kc + b * ks0 + kvh * ks1;
    const float *vb = vc + b * ks0 + kvh * ks1;
    const int total = P + dep;            // visible tokens: prefix then the path (dep <= D_max < W)
    const int ks2_32 = static_cast<int>(ks2);
    // slot of the lane's token in chunk t0 (-1 past the visible tokens); path entry i is
    // a3[i / 64] of lane i % 64
    auto slot_of = [&](int t0) {
        const int idx = t0 + lane;
        const int i = min(max(idx - P, 0), 191), src = (i & 63) << 2;
        const int a0 = __builtin_amdgcn_ds_bpermute(src, a3[0]);
        const int a1 = __builtin_amdgcn_ds_bpermute(src, a3[1]);
        const int a2 = __builtin_amdgcn_ds_bpermute(src, a3[2]);
        const int a = i < 64 ? a0 : i < 128 ? a1 : a2;
        return idx < P ? idx : (idx < total ? P + a - 1 : -1);
    };
    float m = -INFINITY, l = 0.f, acc[DV];
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[e] = 0.f;
    for (int t0 = wv * 64; t0 < total; t0 += kFw * 64) {
        const int cur = slot_of(t0);
        const int n = min(64, total - t0);
        // this chunk's K row (one token per lane) and its first batch of V rows, all issued
        // before any is used
        float4 kv[D / 4];
        {
            const float4 *kr = reinterpret_cast<const float4 *>(kb + static_cast<int64_t>(cur < 0 ? 0 : cur) * ks2);
#pragma unroll
            for (int e = 0; e < D / 4; ++e) kv[e] = kr[e];
        }
        float vv[kBatch][DV];
        auto load_v = [&](int u0) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int t = u0 + u < n ? u0 + u : n - 1;         // padding lanes repeat a row, weight 0
                const int sl = __builtin_amdgcn_readlane(cur, t);
                const float *vr = vb + static_cast<uint32_t>(sl * ks2_32);     // slot * stride < 2^31 (host-checked)
#pragma unroll
                for (int e = 0; e < DV; ++e) vv[u][e] = vr[lane + 64 * e];
            }
        };
        load_v(0);
        float s = -INFINITY;
        if (cur >= 0) {
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < D / 4; ++e) {
                dot = fmaf(qv[e].x, kv[e].x, dot);
                dot = fmaf(qv[e].y, kv[e].y, dot);
                dot = fmaf(qv[e].z, kv[e].z, dot);
                dot = fmaf(qv[e].w, kv[e].w, dot);
            }
            s = dot * scale;
        }
        const float mnew = fmaxf(m, tmv::wave_max(s));
        const float alpha = expf(m - mnew);
        const float p = cur >= 0 ? expf(s - mnew) : 0.f;
        l = l * alpha + tmv::wave_sum(p);
#pragma unroll
        for (int e = 0; e < DV; ++e) acc[e] *= alpha;
        for (int u0 = 0; u0 < n; u0 += kBatch) {
            if (u0 > 0) load_v(u0);
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const float pu = u0 + u < n ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p), u0 + u)) : 0.f;
#pragma unroll
                for (int e = 0; e < DV; ++e) acc[e] = fmaf(pu, vv[u][e], acc[e]);
            }
        }
        m = mnew;
    }
    // the four waves' (max, sum, weighted V) merged in LDS; a wave without a chunk holds
    // (-inf, 0, 0) and contributes nothing
    if (lane == 0) {
        red_ml[wv][0] = m;
        red_ml[wv][1] = l;
    }
#pragma unroll
    for (int e = 0; e < DV; ++e) red_acc[wv][lane + 64 * e] = acc[e];
    __syncthreads();
    if (wv != 0) return;
    float mt = red_ml[0][0];
#pragma unroll
    for (int w = 1; w < kFw; ++w) mt = fmaxf(mt, red_ml[w][0]);
    float lt = 0.f, at[DV];
#pragma unroll
    for (int e = 0; e < DV; ++e) at[e] = 0.f;
#pragma unroll
    for (int w = 0; w < kFw; ++w) {
        const float c = red_ml[w][0] == -INFINITY ? 0.f : expf(red_ml[w][0] - mt);
        lt += c * red_ml[w][1];
#pragma unroll
        for (int e = 0; e < DV; ++e) at[e] += c * red_acc[w][lane + 64 * e];
    }
    const float inv = 1.f / lt;
#pragma unroll
    for (int e = 0; e < DV; ++e) o[lane + 64 * e] = at[e] * inv;
}

template <int D, int WR>
void launch_bf16(const AttnPlan &p, hipStream_t s, int M_max, int D_max, int Hq, int Hkv,
                 const void *q, const int64_t *qs, const void *k, const void *v, const int64_t *kvs,
                 int L_cap, const int32_t *P, const int32_t *n, const int32_t *anc, const int32_t *dep,
                 int32_t *status, float scale, void *out, const int64_t *os, void *ws, size_t off_o, size_t off_stats,
                 const PagedArgs *pg)
{
    char *w = static_cast<char *>(ws);
    uint64_t *cnt = reinterpret_cast<uint64_t *>(w);
    float *stats = reinterpret_cast<float *>(w + off_stats);
    if constexpr (D == 64) {
        float *part = reinterpret_cast<float *>(w + off_o);
        hipLaunchKernelGGL((tree_attn_bf16_stream_kernel<D, WR>), dim3(p.slots * tmv::kXcds), dim3(kWaves * kWave), 0,
                           s, M_max, D_max, Hq, Hkv, static_cast<const uint16_t *>(q), qs[0], qs[1], qs[2],
                           static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), kvs[0], kvs[1],
                           kvs[2], L_cap, P, n, anc, dep, status, scale * kLog2e, static_cast<uint16_t *>(out),
                           os[0], os[1], os[2], stats, part, p.pairs, p.nb, p.splits, p.per_pair);
        // the streaming kernel leaves its split partials to the merge kernel
        if (p.splits > 1) {
            constexpr int RB = WR * kRowsPerWave;
            const int64_t threads = static_cast<int64_t>(p.pairs) * p.nb * RB * (D / 8);
            hipLaunchKernelGGL((tree_attn_merge_kernel<D, RB>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                               dim3(256), 0, s, M_max, D_max, Hq, Hkv, L_cap, P, n, dep, status,
                               static_cast<uint16_t *>(out), os[0], os[1], os[2], stats, part, p.pairs, p.nb, p.splits);
        }
    } else {
        // the ring kernel merges its splits itself (the last split of a row block to arrive)
        uint16_t *part = reinterpret_cast<uint16_t *>(w + off_o);
        // (Hkv <= 0xffff, Hq / Hkv <= 16 and splits <= 16 are checked or planned)
        const uint32_t geom = static_cast<uint32_t>(Hkv) | (static_cast<uint32_t>(Hq / Hkv) << 16) |
                              (static_cast<uint32_t>(p.splits) << 21) | (static_cast<uint32_t>(p.scatter) << 26);
        const unsigned pgroups = static_cast<unsigned>((p.pairs + tmv::kXcds - 1) / tmv::kXcds);
        const dim3 grid = p.adapt ? dim3(static_cast<unsigned>(p.adapt)) : dim3(tmv::kXcds * p.nb, p.splits, pgroups);
        const PagedArgs pgv = pg ? *pg : PagedArgs{nullptr, 0, 0, 0};
#define TMV_LAUNCH_ATTN1(DEEP, PAGED, ADAPT)                                                               \
        hipLaunchKernelGGL((tree_attn_bf16_kernel<D, WR, DEEP, PAGED, ADAPT>), grid,                      \
                           dim3(kRingWaves * kWave), 0, s, static_cast<const uint16_t *>(k),              \
                           static_cast<const uint16_t *>(v), P, n, static_cast<uint32_t>(kvs[0] / 8),     \
                           static_cast<uint32_t>(kvs[1] / 8), static_cast<uint32_t>(kvs[2] / 8), L_cap,   \
                           p.pairs, geom, M_max, D_max, p.nb, static_cast<const uint16_t *>(q), qs[0],    \
                           qs[1], qs[2], anc, dep, status, scale * kLog2e, static_cast<uint16_t *>(out),   \
                           os[0], os[1], os[2], stats, part, cnt, pgv)
#define TMV_LAUNCH_ATTN(DEEP, PAGED)                                                                       \
        do {                                                                                               \
            if (p.adapt) TMV_LAUNCH_ATTN1(DEEP, PAGED, true);                                              \
            else TMV_LAUNCH_ATTN1(DEEP, PAGED, false);                                                     \
        } while (0)
        if (pg) {
            if (D_max + 1 > kAncBatch) TMV_LAUNCH_ATTN(true, true);
            else TMV_LAUNCH_ATTN(false, true);
        } else {
            if (D_max + 1 > kAncBatch) TMV_LAUNCH_ATTN(true, false);
            else TMV_LAUNCH_ATTN(false, false);
        }
#undef TMV_LAUNCH_ATTN
#undef TMV_LAUNCH_ATTN1
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// the bf16 kernels for the plan's row-group width (pg: block table of a paged cache, d128 only)
void dispatch_bf16(const AttnPlan &p, int d, hipStream_t s, int M_max, int D_max, int Hq, int Hkv, const void *q,
                   const int64_t *qs, const void *k, const void *v, const int64_t *kvs, int L_cap, const int32_t *P,
                   const int32_t *n, const int32_t *anc, const int32_t *dep, int32_t *status, float scale, void *out,
                   const int64_t *os, void *ws, size_t off_o, size_t off_stats, const PagedArgs *pg)
{
#define TMV_DISPATCH(DD, WRR) \
    launch_bf16<DD, WRR>(p, s, M_max, D_max, Hq, Hkv, q, qs, k, v, kvs, L_cap, P, n, anc, dep, status, scale, out, os, \
                         ws, off_o, off_stats, pg)
    if (d == 128) {
        if (p.wr == 8) TMV_DISPATCH(128, 8);
        else if (p.wr == 4) TMV_DISPATCH(128, 4);
        else TMV_DISPATCH(128, 2);
    } else {
        if (p.wr == 4) TMV_DISPATCH(64, 4);
        else TMV_DISPATCH(64, 1);
    }
#undef TMV_DISPATCH
}

// the plan's workspace and grid fit the kernels' 32-bit offsets
bool plan_fits(const AttnPlan &p, int d) {
    const int64_t part_rows = static_cast<int64_t>(p.pairs) * p.nb * p.splits * p.rb;
    // (ring kernel grid: (8 nb, splits, ceil(pairs / 8)); streaming kernel: 8 slots)
    // (a scattered plan needs whole XCD groups of pairs and split row blocks of the ring kernel)
    if (p.scatter && (d != 128 || p.adapt || p.splits < 2 || p.pairs % tmv::kXcds != 0)) return false;
    return part_rows * d * 4 < (int64_t(1) << 31) && static_cast<int64_t>(p.slots) * tmv::kXcds <= 0x7fffffff &&
           (p.pairs + tmv::kXcds - 1) / tmv::kXcds <= 65535;
}

size_t attention_workspace(int dtype, int B, int M_max, int Hq, int Hkv, int d, int L_cap, int force_rows,
                           int force_splits)
{
    if (dtype != TMV_BF16 || B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || L_cap < 1 || (d != 64 && d != 128))
        return 256;
    const AttnPlan p = make_plan(B, M_max, Hq, Hkv, L_cap, d, device_cus(), force_rows, force_splits);
    return plan_bytes(p, d, nullptr);
}

int attention(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d, const void *q, const int64_t *q_stride,
              const void *k_cache, const void *v_cache, const int64_t *kv_stride, int L_cap,
              const int32_t *prefix_len, const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
              int32_t *status, float scale, void *out, const int64_t *o_stride, int force_rows, int force_splits,
              void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != TMV_F32 && dtype != TMV_BF16) return TMV_ERR_ARG;
    if (B < 0 || M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128) return TMV_ERR_ARG;
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq / Hkv > 16) return TMV_ERR_ARG;
    if (d != 64 && d != 128) return TMV_ERR_ARG;
    if (L_cap < 1) return TMV_ERR_ARG;
    if (!q_stride || !kv_stride || !o_stride) return TMV_ERR_ARG;
    if (B == 0 || M_max == 0) return TMV_OK;
    if (!q || !k_cache || !v_cache || !prefix_len || !n_nodes || !anc || !depth || !status || !out)
        return TMV_ERR_ARG;
    for (int i = 0; i < 3; ++i)
        if (q_stride[i] < 0 || kv_stride[i] < 0 || o_stride[i] < 0) return TMV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == TMV_F32) {
        const int64_t blocks = static_cast<int64_t>(B) * M_max * Hq;       // one workgroup per row
        if (blocks > 0x7fffffff) return TMV_ERR_ARG;
        // 16-byte loads of q and K rows need 16-byte aligned rows; slot offsets within a
        // (sequence, head) are 32-bit
        if (!aligned16(q) || !aligned16(k_cache) || ((q_stride[0] | q_stride[1] | q_stride[2] | kv_stride[0] |
                                                       kv_stride[1] | kv_stride[2]) & 3))
            return TMV_ERR_ARG;
        if (static_cast<int64_t>(L_cap) * kv_stride[2] >= (int64_t(1) << 31)) return TMV_ERR_ARG;
#define TMV_LAUNCH_F32(DD)                                                                                       \
        hipLaunchKernelGGL(tree_attn_f32_kernel<DD>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, B, M_max, \
                           D_max, Hq, Hkv, static_cast<const float *>(q), q_stride[0], q_stride[1], q_stride[2],  \
                           static_cast<const float *>(k_cache), static_cast<const float *>(v_cache), kv_stride[0], \
                           kv_stride[1], kv_stride[2], L_cap, prefix_len, n_nodes, anc, depth, status, scale,     \
                           static_cast<float *>(out), o_stride[0], o_stride[1], o_stride[2])
        if (d == 64) TMV_LAUNCH_F32(64);
        else TMV_LAUNCH_F32(128);
#undef TMV_LAUNCH_F32
        return tmv_host::launch_status(hipGetLastError());
    }
    // bf16: 16-byte vector loads need 16-byte aligned rows and head slices
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return TMV_ERR_ARG;
    for (int i = 0; i < 3; ++i)
        if ((q_stride[i] | kv_stride[i] | o_stride[i]) & 7) return TMV_ERR_ARG;
    // the d128 kernel takes the cache strides as 32-bit counts of 16-byte units (they are
    // multiples of 8 elements, checked above) and packs the launch geometry
    for (int i = 0; i < 3; ++i)
        if (kv_stride[i] / 8 > 0xffffffffll) return TMV_ERR_ARG;
    if (Hkv > 0xffff) return TMV_ERR_ARG;
    const AttnPlan p = make_plan(B, M_max, Hq, Hkv, L_cap, d, device_cus(), force_rows, force_splits);
    size_t off_o = 0, off_stats = 0;
    const size_t need = plan_bytes(p, d, &off_o, &off_stats);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TMV_ERR_ARG;
    if (!plan_fits(p, d)) return TMV_ERR_ARG;
    dispatch_bf16(p, d, s, M_max, D_max, Hq, Hkv, q, q_stride, k_cache, v_cache, kv_stride, L_cap, prefix_len, n_nodes,
                  anc, depth, status, scale, out, o_stride, workspace, off_o, off_stats, nullptr);
    return tmv_host::launch_status(hipGetLastError());
}

}  // namespace

extern "C" size_t tmv_tree_verify_attention_workspace(int dtype, int B, int M_max, int Hq, int Hkv, int d,
                                                      int L_cap)
{
    return attention_workspace(dtype, B, M_max, Hq, Hkv, d, L_cap, 0, 0);
}

extern "C" int tmv_tree_verify_attention(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                         const void *q, const int64_t *q_stride,
                                         const void *k_cache, const void *v_cache,
                                         const int64_t *kv_stride, int L_cap,
                                         const int32_t *prefix_len, const int32_t *n_nodes,
                                         const int32_t *anc, const int32_t *depth, int32_t *status,
                                         float scale, void *out, const int64_t *o_stride,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    return attention(dtype, B, M_max, D_max, Hq, Hkv, d, q, q_stride, k_cache, v_cache, kv_stride, L_cap, prefix_len,
                     n_nodes, anc, depth, status, scale, out, o_stride, 0, 0, workspace, workspace_bytes, stream);
}

extern "C" size_t tmv_tree_verify_attention_plan_workspace(int dtype, int B, int M_max, int Hq, int Hkv, int d,
                                                           int L_cap, int rows_per_group, int splits)
{
    return attention_workspace(dtype, B, M_max, Hq, Hkv, d, L_cap, rows_per_group, splits);
}

extern "C" int tmv_tree_verify_attention_plan(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                              const void *q, const int64_t *q_stride,
                                              const void *k_cache, const void *v_cache,
                                              const int64_t *kv_stride, int L_cap,
                                              const int32_t *prefix_len, const int32_t *n_nodes,
                                              const int32_t *anc, const int32_t *depth, int32_t *status,
                                              float scale, void *out, const int64_t *o_stride,
                                              int rows_per_group, int splits,
                                              void *workspace, size_t workspace_bytes, void *stream)
{
    return attention(dtype, B, M_max, D_max, Hq, Hkv, d, q, q_stride, k_cache, v_cache, kv_stride, L_cap, prefix_len,
                     n_nodes, anc, depth, status, scale, out, o_stride, rows_per_group, splits, workspace,
                     workspace_bytes, stream);
}

namespace {

size_t paged_workspace(int B, int M_max, int Hq, int Hkv, int d, int page_size, int max_blocks, int force_rows,
                       int force_splits)
{
    if (B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || page_size <= 0 || max_blocks <= 0) return 256;
    const int64_t L_cap = static_cast<int64_t>(page_size) * max_blocks;
    if (L_cap > 0x7fffffff) return 256;
    return plan_bytes(make_plan(B, M_max, Hq, Hkv, static_cast<int>(L_cap), d, device_cus(), force_rows, force_splits),
                      d, nullptr);
}

int paged_attention(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d, const void *q,
                    const int64_t *q_stride, const void *k_pages, const void *v_pages, const int64_t *page_stride,
                    int num_pages, int page_size, const int32_t *block_table, int64_t table_stride, int max_blocks,
                    const int32_t *prefix_len, const int32_t *n_nodes, const int32_t *anc, const int32_t *depth,
                    int32_t *status, float scale, void *out, const int64_t *o_stride, int force_rows,
                    int force_splits, void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != TMV_BF16 || d != 128) return TMV_ERR_ARG;
    if (B < 0 || M_max < 0 || M_max > 128 || D_max < 0 || D_max > 128) return TMV_ERR_ARG;
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || Hq / Hkv > 16 || Hkv > 0xffff) return TMV_ERR_ARG;
    if (page_size < 16 || (page_size & (page_size - 1)) || page_size > (1 << 20)) return TMV_ERR_ARG;
    if (max_blocks < 1 || max_blocks > kMaxPagesLds || num_pages < 1 || table_stride < max_blocks) return TMV_ERR_ARG;
    const int64_t L_cap = static_cast<int64_t>(page_size) * max_blocks;
    if (L_cap > 0x7fffffff) return TMV_ERR_ARG;
    if (!q_stride || !page_stride || !o_stride) return TMV_ERR_ARG;
    if (B == 0 || M_max == 0) return TMV_OK;
    if (!q || !k_pages || !v_pages || !block_table || !prefix_len || !n_nodes || !anc || !depth || !status || !out)
        return TMV_ERR_ARG;
    if (!aligned16(q) || !aligned16(k_pages) || !aligned16(v_pages) || !aligned16(out)) return TMV_ERR_ARG;
    for (int i = 0; i < 3; ++i) {
        if (q_stride[i] < 0 || page_stride[i] < 0 || o_stride[i] < 0) return TMV_ERR_ARG;
        if ((q_stride[i] | page_stride[i] | o_stride[i]) & 7) return TMV_ERR_ARG;
        if (page_stride[i] / 8 > 0xffffffffll) return TMV_ERR_ARG;
    }
    // a chunk's rows are addressed by 32-bit offsets from their page's first row
    if (static_cast<int64_t>(page_size) * page_stride[2] * 2 >= (int64_t(1) << 31)) return TMV_ERR_ARG;
    const AttnPlan p = make_plan(B, M_max, Hq, Hkv, static_cast<int>(L_cap), d, device_cus(), force_rows, force_splits);
    size_t off_o = 0, off_stats = 0;
    const size_t need = plan_bytes(p, d, &off_o, &off_stats);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TMV_ERR_ARG;
    if (!plan_fits(p, d)) return TMV_ERR_ARG;
    int shift = 0;
    while ((1 << shift) < page_size) ++shift;
    const PagedArgs pg{block_table, table_stride, shift, num_pages};
    dispatch_bf16(p, d, static_cast<hipStream_t>(stream), M_max, D_max, Hq, Hkv, q, q_stride, k_pages, v_pages,
                  page_stride, static_cast<int>(L_cap), prefix_len, n_nodes, anc, depth, status, scale, out, o_stride,
                  workspace, off_o, off_stats, &pg);
    return tmv_host::launch_status(hipGetLastError());
}

}  // namespace

extern "C" size_t tmv_tree_verify_attention_paged_workspace(int B, int M_max, int Hq, int Hkv, int d, int page_size,
                                                            int max_blocks)
{
    return paged_workspace(B, M_max, Hq, Hkv, d, page_size, max_blocks, 0, 0);
}

extern "C" int tmv_tree_verify_attention_paged(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                               const void *q, const int64_t *q_stride,
                                               const void *k_pages, const void *v_pages,
                                               const int64_t *page_stride, int num_pages, int page_size,
                                               const int32_t *block_table, int64_t table_stride, int max_blocks,
                                               const int32_t *prefix_len, const int32_t *n_nodes,
                                               const int32_t *anc, const int32_t *depth, int32_t *status,
                                               float scale, void *out, const int64_t *o_stride,
                                               void *workspace, size_t workspace_bytes, void *stream)
{
    return paged_attention(dtype, B, M_max, D_max, Hq, Hkv, d, q, q_stride, k_pages, v_pages, page_stride, num_pages,
                           page_size, block_table, table_stride, max_blocks, prefix_len, n_nodes, anc, depth, status,
                           scale, out, o_stride, 0, 0, workspace, workspace_bytes, stream);
}

extern "C" size_t tmv_tree_verify_attention_paged_plan_workspace(int B, int M_max, int Hq, int Hkv, int d,
                                                                 int page_size, int max_blocks, int rows_per_group,
                                                                 int splits)
{
    return paged_workspace(B, M_max, Hq, Hkv, d, page_size, max_blocks, rows_per_group, splits);
}

extern "C" int tmv_tree_verify_attention_paged_plan(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                                    const void *q, const int64_t *q_stride,
                                                    const void *k_pages, const void *v_pages,
                                                    const int64_t *page_stride, int num_pages, int page_size,
                                                    const int32_t *block_table, int64_t table_stride, int max_blocks,
                                                    const int32_t *prefix_len, const int32_t *n_nodes,
                                                    const int32_t *anc, const int32_t *depth, int32_t *status,
                                                    float scale, void *out, const int64_t *o_stride,
                                                    int rows_per_group, int splits,
                                                    void *workspace, size_t workspace_bytes, void *stream)
{
    return paged_attention(dtype, B, M_max, D_max, Hq, Hkv, d, q, q_stride, k_pages, v_pages, page_stride, num_pages,
                           page_size, block_table, table_stride, max_blocks, prefix_len, n_nodes, anc, depth, status,
                           scale, out, o_stride, rows_per_group, splits, workspace, workspace_bytes, stream);
}

// --------------------------------------------------------------------------- allocation-free call
// Scratch memory of tmv_tree_verify_attention_noalloc: a fixed array on every device the
// library runs on, held until the process ends.  Host code never uses this name as an
// address (on the host it is only a stand-in): the device address comes from
// hipGetSymbolAddress, once per device, and is what the kernels receive.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// zeroes n 32-bit words (the arrival counters; a kernel rather than a memset, so a caller
// may capture the first call in a graph)
__global__ void __launch_bounds__(256) scratch_clear_kernel(uint32_t *p, int n) {
    for (int i = threadIdx.x; i < n; i += 256) p[i] = 0u;
}

// the current device's scratch address; on the device's first call also queues the
// clearing of the counter block on `s` (the array is zero when loaded; the clear makes
// that explicit and costs one tiny launch per device)
int noalloc_scratch(hipStream_t s, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TMV_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TMV_ERR_DEVICE;
        hipLaunchKernelGGL(scratch_clear_kernel, dim3(1), dim3(256), 0, s, static_cast<uint32_t *>(ptr),
                           static_cast<int>(kCounterBytes / 4));
        if (hipGetLastError() != hipSuccess) return TMV_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return TMV_OK;
}

}  // namespace

extern "C" int tmv_tree_verify_attention_noalloc(int dtype, int B, int M_max, int D_max, int Hq, int Hkv, int d,
                                                 const void *q, const int64_t *q_stride,
                                                 const void *k_cache, const void *v_cache,
                                                 const int64_t *kv_stride, int L_cap,
                                                 const int32_t *prefix_len, const int32_t *n_nodes,
                                                 const int32_t *anc, const int32_t *depth, int32_t *status,
                                                 float scale, void *out, const int64_t *o_stride, void *stream)
{
    // the workspace this call needs must fit the fixed scratch (nothing is launched otherwise)
    if (dtype == TMV_BF16 && B > 0 && M_max > 0 &&
        attention_workspace(dtype, B, M_max, Hq, Hkv, d, L_cap, 0, 0) > kNoAllocScratchBytes)
        return TMV_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    const int rc = noalloc_scratch(s, &ws);
    if (rc != TMV_OK) return rc;
    return attention(dtype, B, M_max, D_max, Hq, Hkv, d, q, q_stride, k_cache, v_cache, kv_stride, L_cap, prefix_len,
                     n_nodes, anc, depth, status, scale, out, o_stride, 0, 0, ws, kNoAllocScratchBytes, stream);
}
