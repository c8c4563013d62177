// Split-KV flash-decode for paged K/V on gfx950 (one query token per sequence).
//
// Operation: aclnnFusedInferAttentionScoreV4, "Function" (softmax(scale*QK^T + mask) V,
// per row), decode scenario (one query token); paged K/V per the paged-attention
// constraints of aclnnFusedInferAttentionScoreV3 (token t of sequence b in block
// blockTables[b][t / blockSize], slot t % blockSize); GQA per its numHeads /
// numKeyValueHeads constraint; int8 K/V with per-channel antiquant scales.
//
// Work decomposition (planned on the host): one workgroup = 4 waves = one
// (sequence, kv head, group of <= 16 query heads, range of 32-token tiles).  Each wave
// streams its own contiguous sub-range of tiles with a private online softmax; the four
// wave states are merged in LDS, then written either as the final out/lse (single
// split) or as an un-normalised partial (m, l, O) that the combine kernel merges in a
// fixed order.
//
// Per 32-token tile a wave does, for its 16 packed query heads:
//   S[16 tok x 16 heads] = K_tile . Q^T        2 x (headSize/32) MFMA 16x16x32
//   online softmax on S (in registers; 2 cross-lane steps per reduction)
//   O^T[16 d x 16 heads] += V^T . P^T          8 MFMA 16x16x32 (one per d-phase)
// K rows are MFMA A-operands straight from global memory (each lane reads 16 contiguous
// bytes of one token row).  V is read as 8 token rows x 16 bytes per lane, four whole
// rows per load instruction, and transposed in registers (8x8 of 16-bit values), so no
// LDS traffic is needed on the streaming path.  Tokens are visited in the permuted
// order that makes the S accumulator layout equal the P^T operand layout.
//
// Streaming: every load of a tile is issued from one uniform (scalar) base plus a 32-bit
// per-lane offset, without branches; rows past kvSeqLen are clamped to the last valid
// row (their scores are masked, their V rows zeroed), and the next tile's loads are in
// flight while the current tile is computed.  Block ids are read through the scalar
// cache (one or two s_load per 32-token tile), so the table costs no vector load.
// K/V loads carry the nontemporal hint: each byte is read once per launch, and streaming
// loads keep more HBM bandwidth than loads that allocate normally in the caches (6-7%
// shorter kernels on the long decodes, same results).
//
// FLOAT8_E4M3FN K/V (F8): the one-byte loads of the int8 path; Q (K scale folded in) is
// an f16 operand, normalised by a power of two per head, and each 16-byte K load is
// expanded exactly to f16 (two codes per conversion) as the A operands of two f16 MFMA
// k-steps; V rows are expanded and transposed like the int8 ones.
//
// General int8 antiquant (XQ; aclnnFusedInferAttentionScoreV3, Constraints on the KV
// antiquant parameters), K_hat = scale * (K + offset):
//   per-channel K offset   adds sum_d q'_d o_d (q' = q * sK * qkScale * log2 e) to every
//                          score of a row: out is unchanged, the row max (hence lse and
//                          the split partials' max) carries the constant
//   per-token K            s_j = sK_j * (q'.k_j + oK_j * sum_d q'_d) with q' = q * qkScale
//                          * log2 e (no channel factor)
//   per-token V            P_j is multiplied by sV_j before the PV product (the row sum
//                          keeps P_j), and sum_j P_j sV_j oV_j is added to every O_d
//   per-channel V offset   out_d = sV_d * (O_d / l + oV_d)
// Per-token scales / offsets of a tile: lane l loads entry T + (l & 31) of the K (l < 32)
// or V (l >= 32) tensor with the tile's K rows; the wave passes them through LDS and each
// lane reads its tokens' values back as two 16-byte runs per tensor.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr float kRescaleSlack = 8.0f;   // log2 units a head's max may exceed its reference

// d-chunk (in units of 8 elements) that lane group qg covers at QK k-step kk.
// 16-bit K rows: chunk 4*kk + qg (a load instruction covers 64 contiguous bytes per row).
// int8 K rows: each lane loads 16 bytes = 2 chunks, chunks 2*(qg + 4*(kk/2)) + kk%2.
template <bool I8>
__device__ __forceinline__ int dchunk(int qg, int kk) {
    if constexpr (I8) return 2 * (qg + 4 * (kk >> 1)) + (kk & 1);
    else return 4 * kk + qg;
}

template <int D, bool I8>
struct DecodeTileRegs {
    static constexpr int KN = I8 ? D / 64 : D / 32;   // 16-byte K loads per row
    u32x4 k[2][KN];
    std::conditional_t<I8, u32x2, u32x4> v[8];
    float ta, tb;             // per-token scale / offset of one token (XQ only)
};

// WPH: the item holds 4 kv heads and wave w streams kv head kvh + w over the whole
// tile range (else the 4 waves split the range of one kv head and merge in LDS)
// I8: one-byte K/V with per-channel scales; F8 (with I8): the bytes are FLOAT8_E4M3FN codes
template <int D, bool BF16, bool I8, bool F8, bool ALIBI, bool WPH, bool XQ>
__global__ void __launch_bounds__(256, 2) decode_kernel(DecodeArgs a) {
    static_assert(!XQ || I8, "general antiquant applies to int8 K/V");
    static_assert(!F8 || (I8 && !XQ), "fp8 K/V: one-byte loads, per-channel scales only");
    constexpr int KK = D / 32;                 // QK k-steps
    constexpr int KP = D / 64;                 // int8 16-byte loads per K row
    constexpr bool MBF = BF16 && !I8;          // MFMA element type (int8 path runs in f16)
    constexpr int VCOLS = D / 8;               // lanes (per row) that hold V columns
    constexpr int ESZ = I8 ? 1 : 2;            // bytes per K/V element
    using Tile = DecodeTileRegs<D, I8>;
    using VT = std::conditional_t<I8, u32x2, u32x4>;

    __shared__ float s_m[kDecodeWaves][kHeadPack];
    __shared__ float s_l[kDecodeWaves][kHeadPack];
    __shared__ float s_o[kDecodeWaves][kHeadPack][D];
    // XQ: one tile's per-token values, per wave: scales at [lane], offsets at [64 + lane]
    // (lanes 0..31 hold K's tokens, 32..63 V's)
    __shared__ __attribute__((aligned(16))) float s_tok[kDecodeWaves][128];

    const DecodeItem it = a.items[blockIdx.x];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // the first split of a split sequence hands the combine kernel its item (from device
    // memory, so that the combine's workgroups need no read of the host work list)
    if (it.comb >= 0 && it.t0 == 0 && lane == 0 && (WPH || wave == 0)) {
        const int w = WPH ? wave : 0;
        CombineItem c{};
        c.kvh = it.kvh + w;
        c.hg = it.hg;
        c.slot0 = it.slot + w * it.slot_stride;
        c.nsplit = it.nsplit;
        c.qrow = it.qrow;
        a.comb[it.comb + w] = c;
    }
    const int kvh = it.kvh + (WPH ? wave : 0);  // this wave's kv head
    const int col = lane & 15;                 // packed head (QK/PV column)
    const int qg = lane >> 4;                  // lane group: k-slots 8*qg .. 8*qg+7
    const int hl = it.hg * kHeadPack + col;    // head index within the kv group
    const bool hvalid = hl < a.group;
    const int head = kvh * a.group + (hvalid ? hl : 0);
    const int kvlen = it.kvlen;

    // ------------------------------------------------------------ Q operand
    u32x4 qhi[KK], qlo[KK];
    float s_mul;                               // multiplies the raw MFMA score
    float qsum = 0.0f;                         // XQ, per-token K: sum_d q'_d of head col
    float kconst = 0.0f;                       // XQ, per-channel K offset: sum_d q'_d oK_d
    if constexpr (!I8) {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               static_cast<int64_t>(it.qrow) * a.q_tok_stride +
                               static_cast<int64_t>(head) * a.q_head_stride;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qhi[kk] = hvalid ? *reinterpret_cast<const u32x4*>(qrow + 8 * dchunk<I8>(qg, kk)) : z;
            qlo[kk] = z;
        }
        s_mul = a.scale_log2;
    } else {
        // q' = q * sK * qkScale * log2(e) per channel.  Per head, y = q' * 127 / amax is
        // split into two int8 parts, hi = rint(y) and lo = rint((y - hi) * 256), so that
        // the int8 MFMA gives K.y = acc_hi + acc_lo / 256 (exact integer sums) to about
        // 15 bits relative to the head's largest |q'|; the score in log2 units is then
        // (acc_hi * 256 + acc_lo) * amax / (127 * 256).
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               static_cast<int64_t>(it.qrow) * a.q_tok_stride +
                               static_cast<int64_t>(head) * a.q_head_stride;
        float qf[KP][16];
        float amax = 0.0f;
#pragma unroll
        for (int kp = 0; kp < KP; ++kp) {
            const int d0 = 64 * kp + 16 * qg;       // the lane's 16 channels of k-step kp
#pragma unroll
            for (int h8 = 0; h8 < 2; ++h8) {
                u32x4 raw = {0u, 0u, 0u, 0u};
                if (hvalid) raw = *reinterpret_cast<const u32x4*>(qrow + d0 + 8 * h8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = raw[e >> 1];
                    const float qv = half_to_f32<BF16>((e & 1) ? (w >> 16) : (w & 0xffffu));
                    const int d = d0 + 8 * h8 + e;
                    float sk = 1.0f;                 // per-token K: no channel factor
                    if (!XQ || a.aq.kmode == 0) {
                        if (a.scale_is_f32) {
                            sk = static_cast<const float*>(a.kscale)[kvh * D + d];
                        } else {
                            sk = half_to_f32<BF16>(static_cast<const uint16_t*>(a.kscale)[kvh * D + d]);
                        }
                    }
                    qf[kp][8 * h8 + e] = qv * sk * a.scale_log2;
                    amax = fmaxf(amax, fabsf(qf[kp][8 * h8 + e]));
                    if constexpr (XQ) {
                        if (a.aq.kmode == 1) {
                            qsum += qf[kp][8 * h8 + e];
                        } else if (a.aq.koff != nullptr) {
                            const float ok = a.scale_is_f32
                                ? static_cast<const float*>(a.aq.koff)[kvh * D + d]
                                : half_to_f32<BF16>(static_cast<const uint16_t*>(a.aq.koff)[kvh * D + d]);
                            kconst += qf[kp][8 * h8 + e] * ok;
                        }
                    }
                }
            }
        }
        amax = fmaxf(amax, shfl_xor_f(amax, 16));
        amax = fmaxf(amax, shfl_xor_f(amax, 32));
        if constexpr (XQ) {
            qsum += shfl_xor_f(qsum, 16);
            qsum += shfl_xor_f(qsum, 32);
            kconst += shfl_xor_f(kconst, 16);
            kconst += shfl_xor_f(kconst, 32);
        }
        const bool ok = amax > 0.0f && amax < INFINITY;
        if constexpr (F8) {
            // f16 operand y = q' * 2^ex, |y| < 2^15; k-step kk = 2 kp + h holds channels
            // 64 kp + 16 qg + 8 h .. +7 (the K load layout)
            int ex = 0;
            if (ok) {
                int x;
                frexpf(amax, &x);
                ex = 14 - x;
                ex = ex > 120 ? 120 : (ex < -120 ? -120 : ex);
            }
            const float up = ldexpf(1.0f, ex);
            s_mul = ldexpf(1.0f, -ex);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    qhi[kk][e] = pack2<false>(qf[kk >> 1][8 * (kk & 1) + 2 * e] * up,
                                              qf[kk >> 1][8 * (kk & 1) + 2 * e + 1] * up);
                qlo[kk] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        const float inv = ok ? 127.0f / amax : 0.0f;
        if constexpr (!F8) s_mul = ok ? amax * (1.0f / (127.0f * 256.0f)) : 0.0f;
#pragma unroll
        for (int kp = 0; kp < (F8 ? 0 : KP); ++kp) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                uint32_t hw = 0u, lw = 0u;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float y = qf[kp][4 * w + e] * inv;
                    const float hi = rintf(y);
                    const float lo = fminf(fmaxf(rintf((y - hi) * 256.0f), -127.0f), 127.0f);
                    hw |= (static_cast<uint32_t>(static_cast<int>(hi)) & 0xffu) << (8 * e);
                    lw |= (static_cast<uint32_t>(static_cast<int>(lo)) & 0xffu) << (8 * e);
                }
                qhi[kp][w] = hw;
                qlo[kp][w] = lw;
            }
        }
    }
    float slope2 = 0.0f;
    if constexpr (ALIBI) slope2 = a.slopes[head] * kLog2e;
    const int pos = kvlen - 1;                  // absolute position of the decode query

    // --------------------------------------------------------------- state
    float m_run = -INFINITY;                    // running max (log2 units) of head `col`
    float l_run = 0.0f;                         // this lane's share of the running sum
    float c_run = 0.0f;                         // XQ per-token V offsets: sum P sV oV
    f32x4 acc[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int ntiles = it.t1 - it.t0;
    const int w0 = WPH ? it.t0 : it.t0 + (ntiles * wave) / kDecodeWaves;
    const int w1 = WPH ? it.t1 : it.t0 + (ntiles * (wave + 1)) / kDecodeWaves;
    const int32_t* trow = a.table + static_cast<int64_t>(it.b) * a.table_stride;
    const int bs = a.block_size;
    const char* kpool = static_cast<const char*>(a.k) +
                        static_cast<int64_t>(kvh) * a.k_head_stride * ESZ;
    const char* vpool = static_cast<const char*>(a.v) +
                        static_cast<int64_t>(kvh) * a.v_head_stride * ESZ;
    const int64_t kblk_bytes = a.k_blk_stride * ESZ, vblk_bytes = a.v_blk_stride * ESZ;
    const uint32_t kslot_bytes = static_cast<uint32_t>(a.k_slot_stride * ESZ);
    const uint32_t vslot_bytes = static_cast<uint32_t>(a.v_slot_stride * ESZ);

    const uint32_t vcol = (I8 ? 8u : 16u) * static_cast<uint32_t>(col & (VCOLS - 1));

    // XQ: this lane's per-token tensors (K for lanes 0..31, V for 32..63; a lane whose
    // side is per-channel reads the other side's tensor, which is then per-token)
    const bool ktok = XQ && a.aq.kmode == 1, vtok = XQ && a.aq.vmode == 1;
    const bool tok_loads = ktok || vtok;
    const bool tok_off = XQ && a.aq.koff != nullptr;
    const bool kside = lane < 32 ? ktok : !vtok;
    const float* tok_scale = nullptr;
    const float* tok_offset = nullptr;
    if constexpr (XQ) {
        if (tok_loads) {
            const int64_t row = static_cast<int64_t>(it.b) * (kside ? a.aq.ktok_stride : a.aq.vtok_stride);
            tok_scale = static_cast<const float*>(kside ? a.kscale : a.vscale) + row;
            if (tok_off) tok_offset = static_cast<const float*>(kside ? a.aq.koff : a.aq.voff) + row;
        }
    }

    // Each 16-token half of a 32-token tile lies inside one block (blockSize is a
    // multiple of 16 and tiles start at multiples of 32), so every load of a tile uses a
    // uniform base: K row m and V rows r/4 == h read from half h.  Block ids are scalar
    // loads (constant address space: they do not count against vector-load waits).
    using ctab_t = const __attribute__((address_space(4))) int32_t*;
    const ctab_t ctab = reinterpret_cast<ctab_t>(reinterpret_cast<uintptr_t>(trow));
    struct TileBase {
        int T;
        int lim[2];                  // last valid row inside each half (clamp)
        const char* kb[2];           // row 0 of each half
        const char* vb[2];
    };
    auto tile_base = [&](int tile) -> TileBase {
        TileBase b;
        b.T = tile * kDecodeTile;
        const int t0 = b.T, t1 = b.T + 16;
        const int blk0 = t0 / bs, blk1 = t1 / bs;
        const int e0 = ctab[blk0];
        const bool h1 = t1 < kvlen;                   // second half has a valid row
        const int e1 = (h1 && blk1 != blk0) ? ctab[blk1] : e0;
        const int s0 = t0 - blk0 * bs;
        b.kb[0] = kpool + static_cast<int64_t>(e0) * kblk_bytes + static_cast<int64_t>(s0) * kslot_bytes;
        b.vb[0] = vpool + static_cast<int64_t>(e0) * vblk_bytes + static_cast<int64_t>(s0) * vslot_bytes;
        b.lim[0] = min(15, kvlen - 1 - t0);
        if (h1) {
            const int s1 = t1 - blk1 * bs;
            b.kb[1] = kpool + static_cast<int64_t>(e1) * kblk_bytes + static_cast<int64_t>(s1) * kslot_bytes;
            b.vb[1] = vpool + static_cast<int64_t>(e1) * vblk_bytes + static_cast<int64_t>(s1) * vslot_bytes;
            b.lim[1] = min(15, kvlen - 1 - t1);
        } else {                                      // whole half past kvlen: re-read row kvlen-1
            b.kb[1] = b.kb[0] + static_cast<int64_t>(b.lim[0]) * kslot_bytes;
            b.vb[1] = b.vb[0] + static_cast<int64_t>(b.lim[0]) * vslot_bytes;
            b.lim[1] = 0;
        }
        return b;
    };
    // per-lane byte offsets inside a half: K row `col`, lane group qg's 16-byte chunk(s);
    // V rows 4*qg + (r&3), columns 8*col (in-bounds alias col&(VCOLS-1) when D = 64)
    const uint32_t kqg = 16u * static_cast<uint32_t>(qg);
    auto issue_k = [&](Tile& t, const TileBase& b) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const uint32_t ro = static_cast<uint32_t>(min(col, b.lim[m])) * kslot_bytes + kqg;
#pragma unroll
            for (int i = 0; i < Tile::KN; ++i)
                t.k[m][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b.kb[m] + (ro + 64u * i)));
        }
        if constexpr (XQ) {
            if (tok_loads) {
                // clamp to the sequence's last token (entries past kvSeqLen may not exist)
                const int tk = min(b.T + (lane & 31), max(kvlen - 1, 0));
                t.ta = tok_scale[tk];
                if (tok_off) t.tb = tok_offset[tk];
            }
        }
    };
    auto issue_v = [&](Tile& t, const TileBase& b) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int h = r >> 2;
            const uint32_t ro = static_cast<uint32_t>(min(4 * qg + (r & 3), b.lim[h])) * vslot_bytes + vcol;
            t.v[r] = __builtin_nontemporal_load(reinterpret_cast<const VT*>(b.vb[h] + ro));
        }
    };

    // Process the tile held in `t` (addressed by `cur`) and refill `t` with the tile two
    // ahead (`next`): its K loads are issued right after the QK MFMAs consume K, its V
    // loads right after the transpose consumes V, so two tiles are always in flight.
    auto step = [&](Tile& t, const TileBase& cur, const TileBase& next) {
        const int T = cur.T;
        // XQ: the scores of this lane are tokens 16m + 4qg + r (m, r < 4) of the tile, so
        // after the lanes put their loaded values into the wave's LDS slots each lane reads
        // its K and V values back as 16-byte runs (LDS work of one wave runs in order)
        float tk_s[8], tk_o[8], pv_s[8], pv_o[8];
        if constexpr (XQ) {
            if (tok_loads) {
                float* st = s_tok[wave];
                st[lane] = t.ta;
                if (tok_off) st[64 + lane] = t.tb;
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int j = 16 * m + 4 * qg;
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 ks = ktok ? *reinterpret_cast<const f32x4*>(st + j) : z;
                    const f32x4 ko = ktok && tok_off ? *reinterpret_cast<const f32x4*>(st + 64 + j) : z;
                    const f32x4 vs = vtok ? *reinterpret_cast<const f32x4*>(st + 32 + j) : z;
                    const f32x4 vo = vtok && tok_off ? *reinterpret_cast<const f32x4*>(st + 96 + j) : z;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        tk_s[4 * m + r] = ks[r];
                        tk_o[4 * m + r] = ko[r];
                        pv_s[4 * m + r] = vs[r];
                        pv_o[4 * m + r] = vo[r];
                    }
                }
            }
        }
        // ---- S = K Q^T, scaled to log2 units, bias
        float s[8];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            f32x4 c;
            if constexpr (!I8) {
                c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) c = mfma16x16x32<MBF>(t.k[m][kk], qhi[kk], c);
            } else if constexpr (F8) {
                c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < KK; ++kk) {
                    const u32x4& raw = t.k[m][kk >> 1];
                    const u32x4 kop = f8x8_to_f16x8(raw[2 * (kk & 1)], raw[2 * (kk & 1) + 1]);
                    c = mfma16x16x32<false>(kop, qhi[kk], c);
                }
            } else {
                i32x4 ch = {0, 0, 0, 0}, cl = {0, 0, 0, 0};
#pragma unroll
                for (int kp = 0; kp < KP; ++kp) {
                    ch = mfma16x16x64_i8(t.k[m][kp], qhi[kp], ch);
                    cl = mfma16x16x64_i8(t.k[m][kp], qlo[kp], cl);
                }
                // |acc_hi| <= 127*127*128, so acc_hi * 256 + acc_lo stays below 2^31
#pragma unroll
                for (int r = 0; r < 4; ++r) c[r] = static_cast<float>(ch[r] * 256 + cl[r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float x = c[r] * s_mul;
                if constexpr (XQ) {
                    if (ktok) x = (x + tk_o[4 * m + r] * qsum) * tk_s[4 * m + r];
                }
                if constexpr (ALIBI) x += slope2 * static_cast<float>(T + 16 * m + 4 * qg + r - pos);
                s[4 * m + r] = x;
            }
        }
        issue_k(t, next);
        if (T + kDecodeTile > kvlen) {
            // last tile of the sequence only (wave-uniform): keys past kvlen; the empty asm
            // keeps the compiler from turning this into selects on every tile
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < 8; ++i)
                if (T + 16 * (i >> 2) + 4 * qg + (i & 3) >= kvlen) s[i] = -INFINITY;
        }
        // ---- online softmax (head `col`; its 32 scores live in 4 lanes x 8) against a
        //      lazy reference m_run: heads whose tile max exceeds it by more than the slack
        //      (or that see their first key) re-base it, rescaling O and l; the rest keep
        //      p <= 2^slack
        float tmax = s[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) tmax = fmaxf(tmax, s[i]);
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 16));
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        const bool grow = tmax > m_run + kRescaleSlack || (m_run == -INFINITY && tmax > -INFINITY);
        if (__any(grow)) {
            const float m_new = grow ? tmax : m_run;
            const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
            l_run *= alpha;
            if constexpr (XQ) c_run *= alpha;
#pragma unroll
            for (int n = 0; n < 8; ++n) acc[n] *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            p[i] = fast_exp2(s[i] - m_use);
            l_run += p[i];
        }
        if constexpr (XQ) {
            if (vtok) {
                // V_hat_j = sV_j (V_j + oV_j): weight P_j sV_j on V_j, and the offset part
                // sum_j P_j sV_j oV_j (rows past kvlen have P = 0)
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    p[i] *= pv_s[i];
                    c_run = fmaf(p[i], pv_o[i], c_run);
                }
            }
        }
        u32x4 pop;
        pop.x = pack2<MBF>(p[0], p[1]);
        pop.y = pack2<MBF>(p[2], p[3]);
        pop.z = pack2<MBF>(p[4], p[5]);
        pop.w = pack2<MBF>(p[6], p[7]);

        // ---- V rows (rows past kvlen, tail tile only, are zeroed) transposed into the
        // PV operands: operand n holds column d = 8*col + n of the 8 rows
        VT vrow[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) vrow[r] = t.v[r];
        if (T + kDecodeTile > kvlen) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const bool ok = T + 16 * (r >> 2) + 4 * qg + (r & 3) < kvlen;
                VT z = {};
                vrow[r] = ok ? vrow[r] : z;      // an int8 / fp8 0 converts to f16 0 exactly
            }
        }
        if constexpr (I8) {
            // ---- O^T += V^T P^T, one half of the converted operands at a time
#pragma unroll
            for (int w = 0; w < 2; ++w) {
                u32x4 vop[4];
                if constexpr (F8) f8_rows_to_f16_cols_half(vrow, w, vop);
                else i8_rows_to_f16_cols_half(vrow, w, vop);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[4 * w + j] = mfma16x16x32<MBF>(vop[j], pop, acc[4 * w + j]);
            }
            issue_v(t, next);
        } else {
            // each operand is built right before its MFMA (fewer live registers); the
            // next V loads follow the last one
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                u32x4 vop;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t x = vrow[2 * i][n >> 1], y = vrow[2 * i + 1][n >> 1];
                    vop[i] = (n & 1) ? pack_hi(x, y) : pack_lo(x, y);
                }
                acc[n] = mfma16x16x32<MBF>(vop, pop, acc[n]);
            }
            issue_v(t, next);
        }
    };

    // Two register buffers alternate between even and odd tiles.  Past the end of the
    // range a buffer loads row 0 of block 0 instead (the same few cache lines for every
    // wave, so L2 hits), so that no load sits behind a branch and each wait leaves the
    // later tiles' loads in flight.
    TileBase idle;
    idle.T = 0;
    idle.lim[0] = idle.lim[1] = 0;
    idle.kb[0] = idle.kb[1] = kpool;
    idle.vb[0] = idle.vb[1] = vpool;
    if (w0 < w1) {
        Tile ta, tb;
        TileBase ca = tile_base(w0);
        TileBase cb = (w0 + 1 < w1) ? tile_base(w0 + 1) : idle;
        issue_k(ta, ca);
        issue_v(ta, ca);
        issue_k(tb, cb);
        issue_v(tb, cb);
        for (int tile = w0; tile < w1; tile += 2) {
            const TileBase na = (tile + 2 < w1) ? tile_base(tile + 2) : idle;
            step(ta, ca, na);
            ca = na;
            if (tile + 1 >= w1) break;
            const TileBase nb = (tile + 3 < w1) ? tile_base(tile + 3) : idle;
            step(tb, cb, nb);
            cb = nb;
        }
    }

    // per-channel V scale (and offset) of channel d of kv head c
    auto vchan = [&](int c, int d, bool f32, const void* src) -> float {
        return f32 ? static_cast<const float*>(src)[c * D + d]
                   : half_to_f32<BF16>(static_cast<const uint16_t*>(src)[c * D + d]);
    };
    const bool vscale_f32 = XQ ? a.aq.vscale_is_f32 != 0 : a.scale_is_f32 != 0;
    const bool voff_chan = XQ && !vtok && a.aq.voff != nullptr;
    float c_tot = 0.0f;                         // XQ per-token V offsets, whole head
    if constexpr (XQ) {
        c_tot = c_run + shfl_xor_f(c_run, 16);
        c_tot += shfl_xor_f(c_tot, 32);
    }

    if constexpr (WPH) {
        // ---------------------------------------- each wave owns its kv head's result
        float L = l_run;
        L += shfl_xor_f(L, 16);
        L += shfl_xor_f(L, 32);
        const float M = m_run + kconst;
        const int slot = it.slot < 0 ? -1 : it.slot + wave * it.slot_stride;
        const int geff = a.group;                  // <= 16 in this mode
        if (!hvalid) return;
        const int out_head = kvh * a.group + hl;
        // acc[n][r] = O[head col][d = 32*qg + 8*r + n]
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int d0 = 32 * qg + 8 * r;
            if (d0 >= D) continue;
            float o[8];
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                o[n] = acc[n][r];
                if constexpr (I8) {
                    if (vtok) {
                        o[n] += c_tot;
                    } else {
                        const float sv = vchan(kvh, d0 + n, vscale_f32, a.vscale);
                        if (voff_chan) o[n] = fmaf(vchan(kvh, d0 + n, vscale_f32, a.aq.voff), L, o[n]);
                        o[n] *= sv;
                    }
                }
            }
            if (slot < 0) {
                const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
                u32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = pack2<BF16>(o[2 * i] * inv, o[2 * i + 1] * inv);
                uint16_t* orow = static_cast<uint16_t*>(a.out) +
                                 static_cast<int64_t>(it.qrow) * a.out_tok_stride +
                                 static_cast<int64_t>(out_head) * a.out_head_stride;
                *reinterpret_cast<u32x4*>(orow + d0) = w;
            } else {
                float* po = a.part_o + (static_cast<int64_t>(slot) * geff + hl) * D + d0;
                *reinterpret_cast<f32x4*>(po) = f32x4{o[0], o[1], o[2], o[3]};
                *reinterpret_cast<f32x4*>(po + 4) = f32x4{o[4], o[5], o[6], o[7]};
            }
        }
        if (qg == 0) {
            if (slot < 0) {
                if (a.lse != nullptr)
                    a.lse[static_cast<int64_t>(it.qrow) * a.lse_tok_stride + out_head] =
                        (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : INFINITY;
            } else {
                const int64_t sl = static_cast<int64_t>(slot) * geff + hl;
                a.part_ml[2 * sl] = M;
                a.part_ml[2 * sl + 1] = L;
            }
        }
        return;
    }

    // ------------------------------------------------ merge the 4 wave states
    float l_tot = l_run;
    l_tot += shfl_xor_f(l_tot, 16);
    l_tot += shfl_xor_f(l_tot, 32);
    if (qg == 0) {
        s_m[wave][col] = m_run + kconst;
        s_l[wave][col] = l_tot;
    }
    // acc[n][r] = O[head col][d = 32*qg + 8*r + n]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int d = 32 * qg + 8 * r + n;
            if (d < D) s_o[wave][col][d] = acc[n][r] + c_tot;
        }
    }
    __syncthreads();

    const int geff = a.group < kHeadPack ? a.group : kHeadPack;
    for (int e = threadIdx.x; e < geff * D; e += blockDim.x) {
        const int h = e / D, d = e - (e / D) * D;
        const int hlocal = it.hg * kHeadPack + h;
        if (hlocal >= a.group) continue;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kDecodeWaves; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.0f, O = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kDecodeWaves; ++w) {
                const float f = fast_exp2(s_m[w][h] - M);
                L += s_l[w][h] * f;
                O += s_o[w][h][d] * f;
            }
        }
        if constexpr (I8) {
            if (!vtok) {
                if (voff_chan) O = fmaf(vchan(it.kvh, d, vscale_f32, a.aq.voff), L, O);
                O *= vchan(it.kvh, d, vscale_f32, a.vscale);
            }
        }
        const int out_head = it.kvh * a.group + hlocal;
        if (it.slot < 0) {
            const float val = (L > 0.0f) ? O / L : 0.0f;
            uint16_t* orow = static_cast<uint16_t*>(a.out) +
                             static_cast<int64_t>(it.qrow) * a.out_tok_stride +
                             static_cast<int64_t>(out_head) * a.out_head_stride;
            orow[d] = static_cast<uint16_t>(f32_to_half<BF16>(val));
            if (d == 0 && a.lse != nullptr) {
                a.lse[static_cast<int64_t>(it.qrow) * a.lse_tok_stride + out_head] =
                    (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : INFINITY;
            }
        } else {
            const int64_t sl = static_cast<int64_t>(it.slot) * geff + h;
            a.part_o[sl * D + d] = O;
            if (d == 0) {
                a.part_ml[2 * sl] = M;
                a.part_ml[2 * sl + 1] = L;
            }
        }
    }
}

// Merge the nsplit partials of one (sequence, kv head, head group) in slot order.
template <int D, bool BF16>
__global__ void __launch_bounds__(256) combine_kernel(CombineArgs a) {
    // one thread per output element: item blockIdx.x / per_item, element
    // (blockIdx.x % per_item) * 256 + threadIdx.x of its geff x D block
    const int per_item = a.blocks_per_item;
    const CombineItem it = a.items[blockIdx.x / per_item];
    const int geff = a.group < kHeadPack ? a.group : kHeadPack;
    const int e = (blockIdx.x % per_item) * 256 + threadIdx.x;
    if (e >= geff * D) return;
    const int h = e / D, d = e - (e / D) * D;
    const int hlocal = it.hg * kHeadPack + h;
    if (hlocal >= a.group) return;
    const float* ml = a.part_ml + 2 * (static_cast<int64_t>(it.slot0) * geff + h);
    const float* po = a.part_o + (static_cast<int64_t>(it.slot0) * geff + h) * D + d;
    const int64_t ml_step = 2 * geff, o_step = static_cast<int64_t>(geff) * D;
    const int ns = it.nsplit;
    float M = -INFINITY, L = 0.0f, O = 0.0f;
    constexpr int kMaxLoaded = 8;
    if (ns <= kMaxLoaded) {
        // every split's (m, l, o) is loaded before any is used: one memory round trip
        float pm[kMaxLoaded], pl[kMaxLoaded], pv[kMaxLoaded];
#pragma unroll
        for (int s = 0; s < kMaxLoaded; ++s) {
            if (s < ns) {
                pm[s] = ml[s * ml_step];
                pl[s] = ml[s * ml_step + 1];
                pv[s] = po[s * o_step];
            }
        }
#pragma unroll
        for (int s = 0; s < kMaxLoaded; ++s)
            if (s < ns) M = fmaxf(M, pm[s]);
        if (M != -INFINITY) {
#pragma unroll
            for (int s = 0; s < kMaxLoaded; ++s) {
                if (s < ns) {
                    const float f = fast_exp2(pm[s] - M);
                    L += pl[s] * f;
                    O += pv[s] * f;
                }
            }
        }
    } else {
        // the same sums in the same (ascending) split order, two passes
#pragma unroll 8
        for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[s * ml_step]);
        if (M != -INFINITY) {
#pragma unroll 4
            for (int s = 0; s < ns; ++s) {
                const float f = fast_exp2(ml[s * ml_step] - M);
                L += ml[s * ml_step + 1] * f;
                O += po[s * o_step] * f;
            }
        }
    }
    const int out_head = it.kvh * a.group + hlocal;
    const float val = (L > 0.0f) ? O / L : 0.0f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) +
                     static_cast<int64_t>(it.qrow) * a.out_tok_stride +
                     static_cast<int64_t>(out_head) * a.out_head_stride;
    orow[d] = static_cast<uint16_t>(f32_to_half<BF16>(val));
    if (d == 0 && a.lse != nullptr) {
        a.lse[static_cast<int64_t>(it.qrow) * a.lse_tok_stride + out_head] =
            (L > 0.0f) ? (M + fast_log2(L)) * kLn2 : INFINITY;
    }
}

template <int D, bool BF16, bool I8, bool F8, bool XQ>
void launch_decode_x(const DecodeArgs& a, int n_items, hipStream_t stream, hipEvent_t t0,
                     hipEvent_t t1) {
    const bool alibi = a.mask_type == PA_MASK_ALIBI;
    if (a.wave_heads) {
        if (alibi) launch_256(decode_kernel<D, BF16, I8, F8, true, true, XQ>, n_items, stream, t0, t1, a);
        else launch_256(decode_kernel<D, BF16, I8, F8, false, true, XQ>, n_items, stream, t0, t1, a);
    } else {
        if (alibi) launch_256(decode_kernel<D, BF16, I8, F8, true, false, XQ>, n_items, stream, t0, t1, a);
        else launch_256(decode_kernel<D, BF16, I8, F8, false, false, XQ>, n_items, stream, t0, t1, a);
    }
}

template <int D, bool BF16, bool I8, bool F8>
hipError_t launch_decode_t(const DecodeArgs& a, int n_items, hipStream_t stream, hipEvent_t t0,
                           hipEvent_t t1) {
    if constexpr (I8 && !F8) {
        if (a.aq.extended) {
            launch_decode_x<D, BF16, true, false, true>(a, n_items, stream, t0, t1);
            return hipGetLastError();
        }
    }
    launch_decode_x<D, BF16, I8, F8, false>(a, n_items, stream, t0, t1);
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, int n_items, bool bf16, bool i8, bool f8,
                           hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    if (f8) return bf16 ? launch_decode_t<D, true, true, true>(a, n_items, stream, t0, t1)
                        : launch_decode_t<D, false, true, true>(a, n_items, stream, t0, t1);
    if (i8) return bf16 ? launch_decode_t<D, true, true, false>(a, n_items, stream, t0, t1)
                        : launch_decode_t<D, false, true, false>(a, n_items, stream, t0, t1);
    return bf16 ? launch_decode_t<D, true, false, false>(a, n_items, stream, t0, t1)
                : launch_decode_t<D, false, false, false>(a, n_items, stream, t0, t1);
}

template <int D, bool BF16>
hipError_t launch_combine_t(const CombineArgs& a, int n_items, hipStream_t stream, hipEvent_t t0,
                            hipEvent_t t1) {
    CombineArgs c = a;
    const int geff = a.group < kHeadPack ? a.group : kHeadPack;
    c.blocks_per_item = (geff * D + 255) / 256;
    launch_256(combine_kernel<D, BF16>, n_items * c.blocks_per_item, stream, t0, t1, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int n_items, int head_size, bool bf16, bool i8,
                         bool f8, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    if (n_items <= 0) return hipSuccess;
    if (head_size == 128) return launch_decode_d<128>(a, n_items, bf16, i8, f8, stream, t0, t1);
    return launch_decode_d<64>(a, n_items, bf16, i8, f8, stream, t0, t1);
}

hipError_t launch_combine(const CombineArgs& a, int n_items, int head_size, bool bf16,
                          hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    if (n_items <= 0) return hipSuccess;
    if (head_size == 128)
        return bf16 ? launch_combine_t<128, true>(a, n_items, stream, t0, t1)
                    : launch_combine_t<128, false>(a, n_items, stream, t0, t1);
    return bf16 ? launch_combine_t<64, true>(a, n_items, stream, t0, t1)
                : launch_combine_t<64, false>(a, n_items, stream, t0, t1);
}

}  // namespace pa
