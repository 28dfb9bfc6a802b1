// verify_attention.hip -- tree-masked attention of a flattened draft tree (gfx950).
//
// Every draft node attends to the committed KV prefix plus its own ancestor path,
// itself included, and to nothing else (EAGLE-Pangu, Chinese technical summary section
// 2.3; Medusa section of "Speculative Decoding Hierarquico: Medusa, EAGLE-2 e
// Multi-Token Prediction").  The pages feed a materialised 4D mask to a fused NPU
// kernel; here each query row's ancestor set is a 128-bit mask built in registers from
// the ancestor table, applied only to the <= M tree columns.
//
// bf16 kernel (MFMA, gfx950):
//   * rows of one KV head = (node, query head in the GQA group), node-major; a wave owns
//     32 rows (two 16-row MFMA tiles) and streams 32-token chunks of K and V straight
//     from HBM into registers in MFMA operand layout -- no LDS in the main loop.
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16 leaves each lane holding scores of ONE
//     query row for 8 tokens; those 8 tokens are exactly the lane's slice of the B
//     operand of O^T = V^T P^T, so probabilities never move between lanes.  The token
//     order inside a chunk and the head-dim order inside a tile are permuted (the
//     contraction does not care) so that every K/V load is a contiguous 16-byte read
//     and every V load instruction covers whole 256-byte rows.
//   * online softmax in base 2 (log2 e folded into the scale), row max across the four
//     lanes holding a row via two xor-shuffles; the row sum is kept per lane and reduced
//     once at the end.
//   * a workgroup has 4 waves: either all on the same 32 rows splitting the chunks
//     (WR = 1, combined in LDS) or on 4 different row tiles sharing the chunks through
//     the cache (WR = 4).  Token ranges are further split across workgroups (split-KV);
//     the last workgroup of a split group, found with an atomic ticket, merges the
//     partials in a fixed order (deterministic) -- one launch per call.
//   * workgroup ids are laid out so that every workgroup of one (sequence, KV head)
//     lands on the same XCD: the head's K/V goes from HBM into that XCD's L2 once and
//     its partials stay in the same L2.
// fp32 kernel: one wave per (node, query head), plain FMA; used for fp32 caches.
#include <cstdlib>
#include <cstdio>

#include "tmv_device.hpp"

namespace {

using tmv::kWave;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 32;          // tokens per chunk (two 16-token MFMA tiles)
constexpr int kWaves = 4;
constexpr int kRowsPerWave = 32;    // two 16-row tiles

// --------------------------------------------------------------------------- plan
struct AttnPlan {
    int wr;        // waves along rows (1 or 4); the other 4/wr waves split tokens
    int rb;        // rows per workgroup = wr * 32
    int nb;        // row blocks per (sequence, kv head)
    int splits;    // token splits per row block
    int pairs;     // B * Hkv
    int per_pair;  // workgroups per pair = nb * splits
    int slots;     // workgroups per XCD (ceil(pairs / 8) * per_pair)
};

AttnPlan make_plan(int B, int M_max, int Hq, int Hkv, int L_cap) {
    AttnPlan p;
    const int g = Hq / Hkv;
    const int rows = M_max * g;
    p.wr = rows >= 256 ? 4 : 1;
    int forced_wr = 0, forced_s = 0;
    if (const char *e = std::getenv("TMV_ATTN_PLAN")) std::sscanf(e, "%d:%d", &forced_wr, &forced_s);
    if (forced_wr == 1 || forced_wr == 4) p.wr = forced_wr;
    p.rb = p.wr * kRowsPerWave;
    p.nb = rows > 0 ? (rows + p.rb - 1) / p.rb : 0;
    p.pairs = B * Hkv;
    const int wt = kWaves / p.wr;
    const long base = static_cast<long>(p.pairs) * p.nb;
    int s = base > 0 ? static_cast<int>((256 + base - 1) / base) : 1;
    const int s_tok = L_cap / (wt * 2 * kChunk);          // >= 2 chunks per wave per split
    if (s > s_tok) s = s_tok;
    if (s > 16) s = 16;
    if (s < 1) s = 1;
    if (forced_s >= 1 && forced_s <= 16) s = forced_s;
    p.splits = s;
    p.per_pair = p.nb * p.splits;
    p.slots = ((p.pairs + tmv::kXcds - 1) / tmv::kXcds) * p.per_pair;
    return p;
}

// workspace layout: [counters: pairs*nb u32, padded to 256 B][stats: pairs*nb*S*rb*2 f32]
//                   [partial O: pairs*nb*S*rb*d f32]
size_t plan_bytes(const AttnPlan &p, int d, size_t *off_stats, size_t *off_o) {
    size_t cnt = static_cast<size_t>(p.pairs) * p.nb * sizeof(uint32_t);
    cnt = (cnt + 255) / 256 * 256;
    if (cnt == 0) cnt = 256;
    const size_t units = static_cast<size_t>(p.pairs) * p.nb * p.splits * p.rb;
    size_t st = p.splits > 1 ? units * 2 * sizeof(float) : 0;
    st = (st + 255) / 256 * 256;
    const size_t o = p.splits > 1 ? units * d * sizeof(float) : 0;
    if (off_stats) *off_stats = cnt;
    if (off_o) *off_o = cnt + st;
    return cnt + st + o;
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const uint16_t *p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

// --------------------------------------------------------------------------- bf16 MFMA kernel
template <int D, int WR>
__global__ void __launch_bounds__(kWaves * kWave)
tree_attn_bf16_kernel(int M_max, int D_max, int Hq, int Hkv,
                      const uint16_t *__restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
                      const uint16_t *__restrict__ kc, const uint16_t *__restrict__ vc,
                      int64_t ks0, int64_t ks1, int64_t ks2, int L_cap,
                      const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
                      const int32_t *__restrict__ anc, const int32_t *__restrict__ depth,
                      int32_t *__restrict__ status, float qk_scale_log2,
                      uint16_t *__restrict__ out, int64_t os0, int64_t os1, int64_t os2,
                      uint32_t *__restrict__ counters, float *__restrict__ ws_stats,
                      float *__restrict__ ws_o,
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
    const int wave = threadIdx.x / kWave;
    const int wr = wave / WT, wt = wave % WT;
    const int c16 = lane & 15, G = lane >> 4;

    const int M = n_nodes[b];
    const int P = prefix_len[b];
    const int R = 1 + M_max, W = D_max + 1;
    int st = status[b];
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
        // no live row in this workgroup: the first split clears the block's output rows
        if (split == 0 && wt == 0) write_zero_rows(row0);
        return;
    }
    const bool wave_live = row0 < Rh;

    // ---- per-lane query fragments and ancestor masks for its two rows
    bf16x8_t qf[2][KS];
    uint64_t mlo[2] = {0, 0}, mhi[2] = {0, 0};
    const int T = P + M;                                  // tokens visible to someone
    if (wave_live) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            int r = row0 + rt * 16 + c16;
            if (r >= Rh) r = Rh - 1;                      // padding row: any live row
            const int j = r / g + 1, gi = r % g;
            const uint16_t *qp = q + b * qs0 + static_cast<int64_t>(j - 1) * qs1 + static_cast<int64_t>(kvh * g + gi) * qs2 + G * (8 * KS);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[rt][ks] = load_bf16x8(qp + ks * 8);
            const int32_t *arow = anc + (static_cast<int64_t>(b) * R + j) * W;
            const int dep = depth[static_cast<int64_t>(b) * R + j];
            for (int k = 0; k < dep; ++k) {
                const int a = arow[k] - 1;                // bit a <-> tree slot P + a
                if (a < 64) mlo[rt] |= 1ull << a; else mhi[rt] |= 1ull << (a - 64);
            }
        }
    }

    // ---- token range of this split (in chunks), interleaved over the WT waves
    const int nchunks = (T + kChunk - 1) / kChunk;
    const int c_begin = static_cast<int>(static_cast<int64_t>(nchunks) * split / splits);
    const int c_end = static_cast<int>(static_cast<int64_t>(nchunks) * (split + 1) / splits);

    const uint16_t *kbase = kc + b * ks0 + kvh * ks1;
    const uint16_t *vbase = vc + b * ks0 + kvh * ks1;

    f32x4_t oacc[2][NT];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[rt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrow[2] = {-INFINITY, -INFINITY}, lrow[2] = {0.f, 0.f};

    // registers of one chunk: K fragments (token t0 + tt*16 + c16, dims G*8*KS + ks*8 .. +8)
    // and V rows (tokens pi(G*8 + j), dims c16*NT .. +NT)
    struct Chunk {
        bf16x8_t kf[2][KS];
        uint32_t vr[8][NT / 2];
    };
    auto load_chunk = [&](Chunk &ch, int c) {
        const int t0 = c * kChunk;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            int t = t0 + tt * 16 + c16;
            if (t > T - 1) t = T - 1;
            const uint16_t *kp = kbase + static_cast<int64_t>(t) * ks2 + G * (8 * KS);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ch.kf[tt][ks] = load_bf16x8(kp + ks * 8);
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            int t = t0 + (jj < 4 ? G * 4 + jj : 16 + G * 4 + (jj - 4));
            if (t > T - 1) t = T - 1;
            const uint16_t *vp = vbase + static_cast<int64_t>(t) * ks2 + c16 * NT;
            if constexpr (NT == 8) {
                const uint4 u = *reinterpret_cast<const uint4 *>(vp);
                ch.vr[jj][0] = u.x; ch.vr[jj][1] = u.y; ch.vr[jj][2] = u.z; ch.vr[jj][3] = u.w;
            } else {
                const uint2 u = *reinterpret_cast<const uint2 *>(vp);
                ch.vr[jj][0] = u.x; ch.vr[jj][1] = u.y;
            }
        }
    };
    auto compute_chunk = [&](const Chunk &ch, int c) {
        const int t0 = c * kChunk;
        // S^T tiles: [token][row]
        f32x4_t s[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.kf[tt][ks], qf[rt][ks], acc, 0, 0, 0);
                s[rt][tt] = acc;
            }
        // scale, mask, online softmax; lane holds row c16 of tile rt, tokens
        // t0 + tt*16 + G*4 + i
        const bool needs_mask = t0 + kChunk > P;
        bf16x8_t pb[2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            float v[8];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = s[rt][tt][i] * qk_scale_log2;
                    if (needs_mask) {
                        const int t = t0 + tt * 16 + G * 4 + i;
                        bool vis = t < P;
                        if (!vis && t < T) {
                            const int a = t - P;
                            vis = a < 64 ? ((mlo[rt] >> a) & 1ull) : ((mhi[rt] >> (a - 64)) & 1ull);
                        }
                        if (!vis) x = -INFINITY;
                    }
                    v[tt * 4 + i] = x;
                }
            float cm = v[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) cm = fmaxf(cm, v[e]);
            cm = fmaxf(cm, __shfl_xor(cm, 16, kWave));
            cm = fmaxf(cm, __shfl_xor(cm, 32, kWave));
            const float mnew = fmaxf(mrow[rt], cm);
            const float mref = mnew == -INFINITY ? 0.f : mnew;
            const float alpha = __builtin_amdgcn_exp2f(mrow[rt] - mref);
            float lsum = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const __bf16 pe = static_cast<__bf16>(__builtin_amdgcn_exp2f(v[e] - mref));
                pb[rt][e] = pe;
                lsum += static_cast<float>(pe);
            }
            lrow[rt] = lrow[rt] * alpha + lsum;
            mrow[rt] = mnew;
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) oacc[rt][nt] *= alpha;
        }
        // O^T += V^T P^T; A operand of dim tile nt = (vr[0][nt], ..., vr[7][nt])
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            uint32_t a4[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const uint32_t x = ch.vr[2 * f][nt >> 1], y = ch.vr[2 * f + 1][nt >> 1];
                a4[f] = (nt & 1) ? hi_pair(x, y) : lo_pair(x, y);
            }
            const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(a4[0], a4[1], a4[2], a4[3]));
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
                oacc[rt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[rt], oacc[rt][nt], 0, 0, 0);
        }
    };

    if (wave_live) {
        // ping-pong register buffers: the next chunk's loads are in flight while the
        // current chunk is computed (the prefetch index is clamped, never out of range)
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
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            lrow[rt] += __shfl_xor(lrow[rt], 16, kWave);
            lrow[rt] += __shfl_xor(lrow[rt], 32, kWave);
        }
    }

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

    // ---- split-KV: publish partials, last workgroup of the group merges
    const int64_t unit = (static_cast<int64_t>(pair) * nb + rbk);          // (pair, row block)
    bool finalize = true;
    if (splits > 1) {
        __shared__ int is_last;
        if (wt == 0) {
            const int64_t base = (unit * splits + split) * RB + wr * kRowsPerWave;
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int rr = rt * 16 + c16;
                float *o = ws_o + (base + rr) * D + G * DG;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i * NT + nt] = oacc[rt][nt][i];
                if (G == 0) {
                    ws_stats[(base + rr) * 2 + 0] = mrow[rt];
                    ws_stats[(base + rr) * 2 + 1] = lrow[rt];
                }
            }
        }
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0) {
            const uint32_t prev = atomicAdd(&counters[unit], 1u);
            is_last = prev == static_cast<uint32_t>(splits - 1);
            if (is_last) atomicExch(&counters[unit], 0u);
        }
        __syncthreads();
        finalize = is_last != 0;
        if (finalize && wt == 0) {
            __threadfence();
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int rr = rt * 16 + c16;
                float mo[16], mt = -INFINITY;
                for (int s2 = 0; s2 < splits; ++s2) {
                    const int64_t base = (unit * splits + s2) * RB + wr * kRowsPerWave;
                    mo[s2 & 15] = s2 == split ? mrow[rt] : ws_stats[(base + rr) * 2];
                    mt = fmaxf(mt, mo[s2 & 15]);
                }
                const float mref = mt == -INFINITY ? 0.f : mt;
                f32x4_t acc[NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                float lt = 0.f;
                for (int s2 = 0; s2 < splits; ++s2) {
                    const int64_t base = (unit * splits + s2) * RB + wr * kRowsPerWave;
                    const float sc = __builtin_amdgcn_exp2f(mo[s2 & 15] - mref);
                    if (s2 == split) {
                        lt += sc * lrow[rt];
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt) acc[nt] += sc * oacc[rt][nt];
                    } else {
                        lt += sc * ws_stats[(base + rr) * 2 + 1];
                        const float *o = ws_o + (base + rr) * D + G * DG;
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                            for (int i = 0; i < 4; ++i) acc[nt][i] += sc * o[i * NT + nt];
                    }
                }
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) oacc[rt][nt] = acc[nt];
                lrow[rt] = lt;
            }
        }
    }
    if (!finalize || wt != 0) return;

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
                w4[h2] = static_cast<uint32_t>(tmv::f32_to_bf16(x0)) | (static_cast<uint32_t>(tmv::f32_to_bf16(x1)) << 16);
            }
            *reinterpret_cast<uint4 *>(o + e) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        }
    }
}

// --------------------------------------------------------------------------- fp32 kernel
// One wave per (sequence, node, query head).  Tokens are visited in chunks of 64 (one per
// lane for the scores); the output is accumulated with lanes over the head dims.
__global__ void __launch_bounds__(256)
tree_attn_f32_kernel(int B, int M_max, int D_max, int Hq, int Hkv, int d,
                     const float *__restrict__ q, int64_t qs0, int64_t qs1, int64_t qs2,
                     const float *__restrict__ kc, const float *__restrict__ vc,
                     int64_t ks0, int64_t ks1, int64_t ks2, int L_cap,
                     const int32_t *__restrict__ prefix_len, const int32_t *__restrict__ n_nodes,
                     const int32_t *__restrict__ anc, const int32_t *__restrict__ depth,
                     int32_t *__restrict__ status, float scale,
                     float *__restrict__ out, int64_t os0, int64_t os1, int64_t os2)
{
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + wv;
    if (item >= static_cast<int64_t>(B) * M_max * Hq) return;
    const int h = static_cast<int>(item % Hq);
    const int j = static_cast<int>((item / Hq) % M_max) + 1;
    const int b = static_cast<int>(item / (static_cast<int64_t>(Hq) * M_max));
    const int g = Hq / Hkv, kvh = h / g;
    const int R = M_max + 1, W = D_max + 1;
    float *o = out + b * os0 + static_cast<int64_t>(j - 1) * os1 + h * os2;

    const int M = n_nodes[b], P = prefix_len[b];
    int st = status[b];
    if (st == TMV_OK && (M < 0 || M > M_max || P < 0 || static_cast<int64_t>(P) + M > L_cap)) {
        st = TMV_ERR_INPUT;
        if (lane == 0 && j == 1 && h == 0) status[b] = TMV_ERR_INPUT;
    }
    const int dep = (st == TMV_OK && j <= M) ? depth[static_cast<int64_t>(b) * R + j] : 0;
    if (dep < 1) {
        for (int e = lane; e < d; e += 64) o[e] = 0.f;
        return;
    }
    const float *qp = q + b * qs0 + static_cast<int64_t>(j - 1) * qs1 + h * qs2;

    const float *kb = kc + b * ks0 + kvh * ks1;
    const float *vb = vc + b * ks0 + kvh * ks1;
    const int32_t *arow = anc + (static_cast<int64_t>(b) * R + j) * W;
    const int total = P + dep;            // visible tokens: prefix then the path
    float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
    for (int t0 = 0; t0 < total; t0 += 64) {
        const int idx = t0 + lane;
        int slot = -1;
        if (idx < P) slot = idx;
        else if (idx < total) slot = P + arow[idx - P] - 1;
        float s = -INFINITY;
        if (slot >= 0) {
            const float *kr = kb + static_cast<int64_t>(slot) * ks2;
            float dot = 0.f;
            for (int e = 0; e < d; ++e) dot = fmaf(qp[e], kr[e], dot);
            s = dot * scale;
        }
        const float mnew = fmaxf(m, tmv::wave_max(s));
        const float alpha = expf(m - mnew);
        const float p = slot >= 0 ? expf(s - mnew) : 0.f;
        l = l * alpha + tmv::wave_sum(p);
        acc0 *= alpha;
        acc1 *= alpha;
        const int n = min(64, total - t0);
        for (int t = 0; t < n; ++t) {
            const float pt = __shfl(p, t, 64);
            const int sl = __shfl(slot, t, 64);
            const float *vr = vb + static_cast<int64_t>(sl) * ks2;
            if (lane < d) acc0 = fmaf(pt, vr[lane], acc0);
            if (lane + 64 < d) acc1 = fmaf(pt, vr[lane + 64], acc1);
        }
        m = mnew;
    }
    const float inv = 1.f / l;
    if (lane < d) o[lane] = acc0 * inv;
    if (lane + 64 < d) o[lane + 64] = acc1 * inv;
}

template <int D, int WR>
void launch_bf16(const AttnPlan &p, hipStream_t s, int M_max, int D_max, int Hq, int Hkv,
                 const void *q, const int64_t *qs, const void *k, const void *v, const int64_t *kvs,
                 int L_cap, const int32_t *P, const int32_t *n, const int32_t *anc, const int32_t *dep,
                 int32_t *status, float scale, void *out, const int64_t *os, void *ws, size_t off_st,
                 size_t off_o)
{
    char *w = static_cast<char *>(ws);
    hipLaunchKernelGGL((tree_attn_bf16_kernel<D, WR>), dim3(p.slots * tmv::kXcds), dim3(kWaves * kWave), 0, s,
                       M_max, D_max, Hq, Hkv, static_cast<const uint16_t *>(q), qs[0], qs[1], qs[2],
                       static_cast<const uint16_t *>(k), static_cast<const uint16_t *>(v), kvs[0], kvs[1], kvs[2],
                       L_cap, P, n, anc, dep, status, scale * kLog2e, static_cast<uint16_t *>(out), os[0], os[1],
                       os[2], reinterpret_cast<uint32_t *>(w), reinterpret_cast<float *>(w + off_st),
                       reinterpret_cast<float *>(w + off_o), p.pairs, p.nb, p.splits, p.per_pair);
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" size_t tmv_tree_verify_attention_workspace(int dtype, int B, int M_max, int Hq, int Hkv, int d,
                                                      int L_cap)
{
    if (dtype != TMV_BF16 || B <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv) return 256;
    const AttnPlan p = make_plan(B, M_max, Hq, Hkv, L_cap);
    return plan_bytes(p, d, nullptr, nullptr);
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
        const int64_t items = static_cast<int64_t>(B) * M_max * Hq;
        const int64_t blocks = (items + 3) / 4;
        if (blocks > 0x7fffffff) return TMV_ERR_ARG;
        hipLaunchKernelGGL(tree_attn_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, B, M_max,
                           D_max, Hq, Hkv, d, static_cast<const float *>(q), q_stride[0], q_stride[1], q_stride[2],
                           static_cast<const float *>(k_cache), static_cast<const float *>(v_cache), kv_stride[0],
                           kv_stride[1], kv_stride[2], L_cap, prefix_len, n_nodes, anc, depth, status, scale,
                           static_cast<float *>(out), o_stride[0], o_stride[1], o_stride[2]);
        return tmv_host::launch_status(hipGetLastError());
    }

    // bf16: 16-byte vector loads need 16-byte aligned rows and head slices
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return TMV_ERR_ARG;
    for (int i = 0; i < 3; ++i)
        if ((q_stride[i] | kv_stride[i] | o_stride[i]) & 7) return TMV_ERR_ARG;
    const AttnPlan p = make_plan(B, M_max, Hq, Hkv, L_cap);
    size_t off_st = 0, off_o = 0;
    const size_t need = plan_bytes(p, d, &off_st, &off_o);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return TMV_ERR_ARG;
    if (static_cast<int64_t>(p.slots) * tmv::kXcds > 0x7fffffff) return TMV_ERR_ARG;

    if (d == 128) {
        if (p.wr == 4) launch_bf16<128, 4>(p, s, M_max, D_max, Hq, Hkv, q, q_stride, k_cache, v_cache, kv_stride, L_cap,
                                           prefix_len, n_nodes, anc, depth, status, scale, out, o_stride, workspace, off_st, off_o);
        else launch_bf16<128, 1>(p, s, M_max, D_max, Hq, Hkv, q, q_stride, k_cache, v_cache, kv_stride, L_cap,
                                 prefix_len, n_nodes, anc, depth, status, scale, out, o_stride, workspace, off_st, off_o);
    } else {
        if (p.wr == 4) launch_bf16<64, 4>(p, s, M_max, D_max, Hq, Hkv, q, q_stride, k_cache, v_cache, kv_stride, L_cap,
                                          prefix_len, n_nodes, anc, depth, status, scale, out, o_stride, workspace, off_st, off_o);
        else launch_bf16<64, 1>(p, s, M_max, D_max, Hq, Hkv, q, q_stride, k_cache, v_cache, kv_stride, L_cap,
                                prefix_len, n_nodes, anc, depth, status, scale, out, o_stride, workspace, off_st, off_o);
    }
    return tmv_host::launch_status(hipGetLastError());
}
