// Paged prefill / prefix-encoder attention on gfx950 (seqLen > 1 queries per sequence).
//
// Operation: aclnnFusedInferAttentionScoreV4, "Function" (softmax(scale*QK^T + mask) V),
// prefill scenario; PrefixEncoder (Definition, Members): the new query tokens of a
// sequence attend over its paged cache of kvSeqLen tokens (cached prefix + new tokens),
// maskType 9 = causal mask generated internally, maskType 3 = ALiBi bias
// slopes[h] * (j - p_i) plus causal, qkScale post-multiplying Q*K^T.  Query i of a
// sequence sits at absolute position p_i = kvSeqLen - seqLen + i.
//
// One workgroup = 4 waves covering `heads` (1, 2 or 4) query heads of one kv group and
// 128 / heads query rows; wave w owns head h + w % heads and 32 rows.  All heads of the
// workgroup read the same K/V, so each key tile is staged in LDS once for all of them.
// Keys are visited in tiles of 64, from the tile holding the last key any of the rows
// can see down to key 0.  Per tile:
//   wave w:      loads keys 16w .. 16w+15 of the tile (one 16-key group always lies in
//                one cache block: a uniform base + constant per-lane offsets) into LDS,
//                K and V both row-major
//   per wave:    S^T[64 keys x 32 rows] = K . Q^T      (D/16 x 2 MFMA 32x32x16)
//                scale, ALiBi bias, causal / tail mask, online softmax in registers
//                (a lane owns one query row; one cross-lane step per reduction), with
//                the row maximum re-based only when it grows by more than 2^8
//                O^T[D x 32 rows] += V^T . P^T          (D/32 x 4 MFMA 32x32x16), the
//                V^T operands read straight from row-major V with the LDS transpose
//                read ds_read_b64_tr_b16
// Q stays in registers as the B operand; LDS is double-buffered so one barrier per key
// tile suffices, and the next tile's global loads are in flight during the MFMA work.
// ALiBi over 16-bit K/V: prefix tiles whose bias alone lies far below the nearest keys'
// are not computed when a Cauchy-Schwarz bound on their scores (the workgroup's largest
// |scaled q| times the tile's largest |k|, plus the tile's largest bias), taken from
// their K rows streamed through registers after the other tiles, shows every weight
// negligible next to its row's largest; a tile the bound does not cover is computed.
// int8 K/V are converted exactly to f16 on the way into LDS; the per-channel K scale is
// folded into Q (kept to ~22 bits as an f16 hi + lo pair), the V scale into the output.
// FLOAT8_E4M3FN K/V take the int8 path with the codes expanded exactly to f16 instead.
// General antiquant (aclnnFusedInferAttentionScoreV3, Constraints on the KV antiquant
// parameters; K_hat = scale * (K + offset)): per-token K or V rows are dequantised on the
// way into LDS, sK_j (K_j + oK_j) rounded to f16; a per-channel K offset adds
// sum_d q'_d oK_d to every score of a row, which only moves the row max (lse); a
// per-channel V offset gives out_d = sV_d (O_d / l + oV_d).
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int BN = kPrefillBN;          // 64 keys per tile
constexpr float kRescaleSlack = 8.0f;   // log2 units a row max may exceed its reference
constexpr float kNegligible = 32.0f;    // log2 units below the reference: weight < 2^-32
// s_waitcnt immediate for vmcnt(0) with expcnt / lgkmcnt left at their maxima (gfx9
// encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16;

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4*j + p supplies the 4 16-bit
// values at its address; lane i of the group receives value i % 4 of lanes
// i / 4, 4 + i / 4, 8 + i / 4, 12 + i / 4 (in that order).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_v4i16)(reinterpret_cast<uintptr_t>(p)));
    return __builtin_bit_cast(u32x2, v);
}

// MASK: 0 = none, 1 = causal, 2 = ALiBi (+ causal), fixed at compile time so that the
// per-score work of each variant holds no run-time selects.
// I8: one-byte K/V (int8, or FLOAT8_E4M3FN codes when F8) with per-channel scales
template <int D, bool BF16, bool I8, bool F8, int MASK>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PrefillArgs a) {
    static_assert(!F8 || I8, "fp8 K/V use the one-byte path");
    constexpr bool MBF = BF16 && !I8;
    constexpr int KS = D / 16;            // QK k-steps (32x32x16)
    constexpr int DT = D / 32;            // PV output row blocks
    // 16-bit K/V go global -> LDS directly into swizzled, unpadded rows; int8 K/V pass
    // through registers (exact conversion to f16) into padded rows
    constexpr bool DIRECT = !I8;
    constexpr int KLD = DIRECT ? D : D + 8;     // K tile LDS row (16-bit elements)
    constexpr int VLD = DIRECT ? D : D + 32;    // V tile LDS row
    constexpr int ESZ = I8 ? 1 : 2;       // bytes per global K/V element
    constexpr int CH = D * ESZ / 16;      // 16-byte chunks per global K/V row
    constexpr int NL = 16 * CH / 64;      // 16-byte loads per lane for a 16-key group
    constexpr int EPC = 16 / ESZ;         // elements per 16-byte chunk

    // K tiles in slots 0 and 1, V tiles in slots 2 and 3 (for 16-bit K/V the four slots
    // are alike)
    __shared__ uint16_t s_kv[2 * BN * KLD + 2 * BN * VLD];
    // far tiles of an ALiBi item: per wave, the smallest largest-score-so-far among its
    // query rows, the largest |s_mul q| among them, and the first and last far tile its
    // rows leave uncovered
    __shared__ float s_mmin[4], s_qmax[4];
    __shared__ int s_frange[2][4];
    auto kbuf = [](int b) { return s_kv + b * (BN * KLD); };
    auto vbuf = [](int b) { return s_kv + 2 * (BN * KLD) + b * (BN * VLD); };

    const PrefillItem it = a.items[blockIdx.x];
    if (it.heads == 0) return;            // padding item of the XCD-ordered list
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int qcol = lane & 31;           // query row of this lane inside the wave
    const int g2 = lane >> 5;             // k-slot half
    const int heads = it.heads;
    const int h = it.h + wave % heads;    // this wave's query head
    const int kvh = it.h / a.group;
    const int64_t kvh_off = static_cast<int64_t>(kvh) * D;      // into the [Hkv, D] scales
    const int kvlen = it.kvlen;
    const int qlen = it.qlen;
    constexpr bool causal = MASK != 0;
    constexpr bool alibi = MASK == 2;
    const int shift = kvlen - qlen;       // p_i = shift + i

    const int wave_q0 = it.qbeg + 32 * (wave / heads);      // first local row of the wave
    const int qi = wave_q0 + qcol;                          // local query row of this lane
    const bool qvalid = qi < qlen;
    const int pos = shift + qi;                             // its absolute position
    const int wave_pmin = shift + wave_q0;                  // lowest position of its rows

    // ---------------------------------------------------------------- Q^T
    u32x4 qhi[KS], qlo[KS];
    float s_mul;
    // general int8 antiquant: per-token sides, and the per-channel K offset's row constant
    const bool ktok = I8 && !F8 && a.aq.kmode == 1, vtok = I8 && !F8 && a.aq.vmode == 1;
    const bool tok_off = I8 && a.aq.koff != nullptr;
    float kconst = 0.0f;
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               static_cast<int64_t>(it.qrow0 + (qvalid ? qi : 0)) * a.q_tok_stride +
                               static_cast<int64_t>(h) * a.q_head_stride;
        if constexpr (!I8) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 z = {0u, 0u, 0u, 0u};
                qhi[ks] = qvalid ? *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * g2) : z;
                qlo[ks] = z;
            }
            s_mul = a.scale_log2;
        } else {
            float qf[KS][8];
            float amax = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int d0 = 16 * ks + 8 * g2;
                u32x4 raw = {0u, 0u, 0u, 0u};
                if (qvalid) raw = *reinterpret_cast<const u32x4*>(qrow + d0);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = raw[e >> 1];
                    const float qv = half_to_f32<BF16>((e & 1) ? (w >> 16) : (w & 0xffffu));
                    float sk = 1.0f;                 // per-token K: dequantised in LDS
                    if (!ktok) {
                        if (a.scale_is_f32) sk = static_cast<const float*>(a.kscale)[kvh_off + d0 + e];
                        else sk = half_to_f32<BF16>(static_cast<const uint16_t*>(a.kscale)[kvh_off + d0 + e]);
                    }
                    qf[ks][e] = qv * sk * a.scale_log2;
                    amax = fmaxf(amax, fabsf(qf[ks][e]));
                    if (!ktok && a.aq.koff != nullptr) {
                        const float ok = a.scale_is_f32
                            ? static_cast<const float*>(a.aq.koff)[kvh_off + d0 + e]
                            : half_to_f32<BF16>(static_cast<const uint16_t*>(a.aq.koff)[kvh_off + d0 + e]);
                        kconst += qf[ks][e] * ok;
                    }
                }
            }
            amax = fmaxf(amax, shfl_xor_f(amax, 32));
            kconst += shfl_xor_f(kconst, 32);
            int ex = 0;
            if (amax > 0.0f && amax < INFINITY) {
                int x;
                frexpf(amax, &x);
                ex = 14 - x;
                ex = ex > 120 ? 120 : (ex < -120 ? -120 : ex);
            }
            const float up = ldexpf(1.0f, ex);
            s_mul = ldexpf(1.0f, -ex);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const float x0 = qf[ks][e] * up, x1 = qf[ks][e + 1] * up;
                    const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
                    const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
                    const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
                    qhi[ks][e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h0)) |
                                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h1)) << 16);
                    qlo[ks][e >> 1] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l0)) |
                                      (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, l1)) << 16);
                }
            }
        }
    }
    const float slope2 = alibi ? a.slopes[h] * kLog2e : 0.0f;
    // ALiBi's within-tile part slope2 * dj (dj = key offset from the tile start) enters
    // the QK accumulator as one extra rank-1 bf16 product per 32-key block:
    // A[key m][k] = dj_m for k = 0..2 (exact), B[k][row] = c = slope2 / s_mul in raw
    // score units, split into three bf16 terms (~24 bits); lanes 32..63 (k = 4..7) hold
    // zeros.  If c is not usable (s_mul ~ 0, i.e. qkScale ~ 0) the row's Q*K term is
    // below f32 resolution next to the bias: the row then takes Q = 0, s_mul = 1.
    u32x2 bias_a[2] = {{0u, 0u}, {0u, 0u}}, bias_b = {0u, 0u};
    if constexpr (alibi) {
        float c = slope2 / s_mul;
        if (!(fabsf(c) < 1e30f)) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qhi[ks] = qlo[ks] = u32x4{0u, 0u, 0u, 0u};
            s_mul = 1.0f;
            c = slope2;
        }
        if (g2 == 0) {
            const uint32_t hi = f32_to_half<true>(c);
            const float r1 = c - half_to_f32<true>(hi);
            const uint32_t mid = f32_to_half<true>(r1);
            const uint32_t lo = f32_to_half<true>(r1 - half_to_f32<true>(mid));
            bias_b = u32x2{hi | (mid << 16), lo};
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const uint32_t d = f32_to_half<true>(static_cast<float>(32 * mt + qcol));
                bias_a[mt] = u32x2{d | (d << 16), d};
            }
        }
    }

    // far tiles of an ALiBi item: the largest |s_mul q| among the wave's query rows (lane l
    // and l ^ 32 hold the two halves of row l % 32), published by the first barrier
    if constexpr (alibi && DIRECT) {
        float ss = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int e = 0; e < 4; ++e) ss = dot2_self<MBF>(qhi[ks][e], ss);
        }
        ss += shfl_xor_f(ss, 32);
        const float qn = wave_max(qvalid ? sqrtf(ss) : 0.0f);
        if (lane == 0) s_qmax[wave] = qn * fabsf(s_mul);
    }

    // ---------------------------------------------------------- tile loads
    // Wave w stages keys 16w .. 16w+15 of each tile.  They lie in one cache block, so
    // the block base is uniform and each lane reads at fixed offsets from it.
    using ctab_t = const __attribute__((address_space(4))) int32_t*;
    const ctab_t ctab = reinterpret_cast<ctab_t>(
        reinterpret_cast<uintptr_t>(a.table + static_cast<int64_t>(it.b) * a.table_stride));
    const int bs = a.block_size;
    const char* kpool = static_cast<const char*>(a.k) + static_cast<int64_t>(kvh) * a.k_head_stride * ESZ;
    const char* vpool = static_cast<const char*>(a.v) + static_cast<int64_t>(kvh) * a.v_head_stride * ESZ;
    const int64_t kblk_bytes = a.k_blk_stride * ESZ, vblk_bytes = a.v_blk_stride * ESZ;
    const int64_t kslot_bytes = a.k_slot_stride * ESZ, vslot_bytes = a.v_slot_stride * ESZ;
    // load i of a lane covers row RPI*i + lane / CH, 16-byte chunk lane % CH of the
    // wave's 16-key group: one 32-bit lane offset, the row step goes into the scalar base
    constexpr int RPI = 64 / CH;          // rows per load instruction
    const int lrow = lane / CH, lch = lane % CH;
    const uint32_t koff = static_cast<uint32_t>(lrow * kslot_bytes) + 16u * lch;
    const uint32_t voff = static_cast<uint32_t>(lrow * vslot_bytes) + 16u * lch;
    // LDS element offsets of the lane's first K / V row (row 16*wave + lrow)
    constexpr int KLW = I8 ? 2 : 1;       // 16-byte LDS stores per loaded chunk
    const int lds_k = (16 * wave + lrow) * KLD + EPC * lch;
    const int lds_v = (16 * wave + lrow) * VLD + EPC * lch;

    u32x4 kreg[NL], vreg[NL];
    float ktok_s[NL], ktok_o[NL], vtok_s[NL], vtok_o[NL];   // per-token values of the rows
    // per-token scale / offset of load i's row of tile jt (token clamped to kvlen - 1)
    auto load_tok = [&](const void* sc, const void* off, int64_t stride, float (&vs)[NL],
                        float (&vo)[NL], int jt) {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int tok = min(jt * BN + 16 * wave + RPI * i + lrow, kvlen - 1);
            const int64_t at = static_cast<int64_t>(it.b) * stride + tok;
            vs[i] = static_cast<const float*>(sc)[at];
            vo[i] = tok_off ? static_cast<const float*>(off)[at] : 0.0f;
        }
    };
    // uniform base of this wave's 16-key group of tile jt (a group wholly past kvlen
    // re-reads the tile's first group: its V rows are zeroed before they reach LDS, its
    // K rows are masked)
    auto group_base = [&](const char* pool, int64_t blk_bytes, int64_t slot_bytes, int jt) {
        const int j0 = jt * BN;
        const int tok0 = (j0 + 16 * wave < kvlen) ? j0 + 16 * wave : j0;
        const int blk = tok0 / bs;
        const int slot0 = tok0 - blk * bs;
        const int e = ctab[blk];
        return pool + e * blk_bytes + slot0 * slot_bytes;
    };
    // every load = uniform base (pinned to SGPRs) + the lane's 32-bit offset (kept 32-bit
    // inside the loop), so that it takes the scalar-base form with no per-load address
    // arithmetic
    using gptr = const __attribute__((address_space(1))) u32x4*;
    auto load_rows = [&](u32x4 (&reg)[NL], const char* base, int64_t slot_bytes, uint32_t off) {
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            uint64_t bi = reinterpret_cast<uintptr_t>(base + i * RPI * slot_bytes);
            asm volatile("" : "+s"(bi));
            reg[i] = *reinterpret_cast<gptr>(bi + off);
        }
    };
    auto load_k = [&](int jt) {
        load_rows(kreg, group_base(kpool, kblk_bytes, kslot_bytes, jt), kslot_bytes, koff);
        if (ktok) load_tok(a.kscale, a.aq.koff, a.aq.ktok_stride, ktok_s, ktok_o, jt);
    };
    auto load_v = [&](int jt) {
        load_rows(vreg, group_base(vpool, vblk_bytes, vslot_bytes, jt), vslot_bytes, voff);
        if (vtok) load_tok(a.vscale, a.aq.voff, a.aq.vtok_stride, vtok_s, vtok_o, jt);
    };
    // 16-byte chunk(s) to LDS; int8 chunks become two f16 chunks (exact)
    auto put = [&](uint16_t* dst, const u32x4& x) {
        if constexpr (!I8) {
            *reinterpret_cast<u32x4*>(dst) = x;
        } else if constexpr (F8) {
            *reinterpret_cast<u32x4*>(dst) = f8x8_to_f16x8(x.x, x.y);
            *reinterpret_cast<u32x4*>(dst + 8) = f8x8_to_f16x8(x.z, x.w);
        } else {
            static_assert(KLW == 2, "int8 chunks expand to two f16 chunks");
            const u32x2 c0 = i8x4_to_f16x4(x.x), c1 = i8x4_to_f16x4(x.y);
            const u32x2 c2 = i8x4_to_f16x4(x.z), c3 = i8x4_to_f16x4(x.w);
            *reinterpret_cast<u32x4*>(dst) = u32x4{c0.x, c0.y, c1.x, c1.y};
            *reinterpret_cast<u32x4*>(dst + 8) = u32x4{c2.x, c2.y, c3.x, c3.y};
        }
    };
    // 16 int8 values -> f16 of sc * (x + of), two 16-byte chunks (per-token rows)
    auto put_tok = [&](uint16_t* dst, const u32x4& x, float sc, float of) {
        if constexpr (I8) {
            uint32_t w[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int lo = static_cast<int8_t>((x[q] >> (16 * h)) & 0xffu);
                    const int hi = static_cast<int8_t>((x[q] >> (16 * h + 8)) & 0xffu);
                    w[2 * q + h] = pack2<false>((static_cast<float>(lo) + of) * sc,
                                                (static_cast<float>(hi) + of) * sc);
                }
            }
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
            *reinterpret_cast<u32x4*>(dst + 8) = u32x4{w[4], w[5], w[6], w[7]};
        }
    };
    auto store_k = [&](int buf) {
        uint16_t* ks = kbuf(buf) + lds_k;
        if (ktok) {
#pragma unroll
            for (int i = 0; i < NL; ++i) put_tok(ks + RPI * i * KLD, kreg[i], ktok_s[i], ktok_o[i]);
            return;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) put(ks + RPI * i * KLD, kreg[i]);
    };
    auto store_v = [&](int buf, int jt) {
        const int j0 = jt * BN;
        if (j0 + BN > kvlen) {
            // tail tile only (wave-uniform): zero the V rows past kvlen; the empty asm
            // keeps the compiler from turning this into selects on every tile
            asm volatile("" ::: "memory");
#pragma unroll
            for (int i = 0; i < NL; ++i)
                if (j0 + 16 * wave + RPI * i + lrow >= kvlen) vreg[i] = u32x4{0u, 0u, 0u, 0u};
        }
        uint16_t* vs = vbuf(buf) + lds_v;
        if (vtok) {
            // rows past kvlen: zero after the dequant (their P is 0; keep them finite)
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const bool live = j0 + 16 * wave + RPI * i + lrow < kvlen;
                put_tok(vs + RPI * i * VLD, vreg[i], live ? vtok_s[i] : 0.0f, vtok_o[i]);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) put(vs + RPI * i * VLD, vreg[i]);
    };

    // ---- direct global -> LDS staging (16-bit K/V).  LDS rows hold D elements with no
    //      padding, and LDS serves 256 bytes (64 banks) per cycle: 16 lanes of a
    //      ds_read_b128, 32 lanes of a transposed ds_read_b64.  The K operand reads take
    //      one chunk of 16 consecutive rows, the transposed V reads 4 chunks of 4 rows,
    //      so 16-byte chunk c of tile row r sits at position c ^ kswz(r) / c ^ vswz(r),
    //      which spreads each of those sets over all 16 chunk positions of a 256-byte
    //      bank line (D = 64 rows pack two to a line).  global_load_lds_dwordx4 writes
    //      lane L's 16 bytes to slot L of a 1 KB run (RPI rows) at the uniform LDS
    //      address in M0, so lane L loads the chunk that belongs at its slot.  Rows past
    //      kvlen re-read row kvlen - 1 (finite values: their V rows meet P = 0, their K
    //      rows are masked).
    auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
    auto vswz = [](int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); };
    using gvoid = __attribute__((address_space(1))) void;
    using lvoid = __attribute__((address_space(3))) void;
    const int bshift = a.block_shift;
    // lane byte offset of load i (source row src relative to the group's base token):
    // the row's slot offset plus the lane's swizzled 16-byte chunk
    auto lane_off = [&](int i, int src, uint32_t slot_bytes, bool is_k) {
        const int r = RPI * i + lrow;                       // LDS row in the group
        const int pos = lch ^ (is_k ? kswz(r) : vswz(r));   // the lane's slot holds
        return static_cast<uint32_t>(src) * slot_bytes + 16u * pos;
    };
    const uint32_t kslot32 = static_cast<uint32_t>(kslot_bytes);
    const uint32_t vslot32 = static_cast<uint32_t>(vslot_bytes);
    // offsets of a full tile (source row = LDS row) are the same for every tile
    uint32_t koff_full[NL], voff_full[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        koff_full[i] = lane_off(i, RPI * i + lrow, kslot32, true);
        voff_full[i] = lane_off(i, RPI * i + lrow, vslot32, false);
    }
    // one 16-key group: base = uniform address of the group's first token, off[i] = the
    // lane's byte offset of load i, dst = LDS row 0 of the group
    auto issue_group = [&](const char* base, uint16_t* dst, int ld, const uint32_t (&off)[NL]) {
        uint64_t bi = reinterpret_cast<uintptr_t>(base);
        asm volatile("" : "+s"(bi));
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            // opaque 32-bit lane offset: the load then takes the scalar-base +
            // 32-bit-offset form with no per-load address arithmetic
            uint32_t o = off[i];
            asm volatile("" : "+v"(o));
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const gvoid*>(bi + o),
                reinterpret_cast<lvoid*>(reinterpret_cast<uintptr_t>(dst + RPI * i * ld)), 16, 0, 0);
        }
    };
    auto load_tile_direct = [&](int buf, int t, bool with_k, bool with_v) {
        const int j0 = t * BN;
        const int g0 = j0 + 16 * wave;
        int gb = g0;
        // block and slot of token gb, shared by K and V: a shift for power-of-two block
        // sizes (a wave-uniform branch), else a division; offsets inside a block fit 32
        // bits (the planner bounds a block's span), block ids are taken as non-negative
        auto bases = [&](const char*& kb, const char*& vb) {
            const int blk = bshift >= 0 ? (gb >> bshift)
                                        : static_cast<int>(static_cast<uint32_t>(gb) /
                                                           static_cast<uint32_t>(bs));
            const uint32_t slot = static_cast<uint32_t>(gb - blk * bs);
            const uint64_t e = static_cast<uint32_t>(ctab[blk]);
            kb = kpool + e * static_cast<uint64_t>(kblk_bytes) + slot * kslot32;
            vb = vpool + e * static_cast<uint64_t>(vblk_bytes) + slot * vslot32;
        };
        const char *kb, *vb;
        if (j0 + BN <= kvlen) {
            bases(kb, vb);
            if (with_k) issue_group(kb, kbuf(buf) + 16 * wave * KLD, KLD, koff_full);
            if (with_v) issue_group(vb, vbuf(buf) + 16 * wave * VLD, VLD, voff_full);
        } else {
            // tail tile (wave-uniform branch): rows past kvlen re-read row kvlen - 1
            asm volatile("" ::: "memory");
            const int last = kvlen - 1;
            gb = g0 <= last ? g0 : last;
            uint32_t ko[NL], vo[NL];
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int src = min(RPI * i + lrow, last - gb);
                ko[i] = lane_off(i, src, kslot32, true);
                vo[i] = lane_off(i, src, vslot32, false);
            }
            bases(kb, vb);
            if (with_k) issue_group(kb, kbuf(buf) + 16 * wave * KLD, KLD, ko);
            if (with_v) issue_group(vb, vbuf(buf) + 16 * wave * VLD, VLD, vo);
        }
    };

    // element offset of 16-byte chunk c of K / V tile row r
    auto kpos = [&](int r, int c) { return r * KLD + 8 * (DIRECT ? (c ^ kswz(r)) : c); };
    auto vpos = [&](int r, int c) { return r * VLD + 8 * (DIRECT ? (c ^ vswz(r)) : c); };

    // transposed-read coordinates: lane group G = lane / 16 covers d half G % 2 and key
    // half g2; inside the group lane 4*jj + pp reads key row jj, columns 4*pp .. 4*pp+3
    const int tr_row = 4 * g2 + ((lane & 15) >> 2);
    const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    // --------------------------------------------------------------- state
    float m_ref = -INFINITY;              // reference row max (log2 units)
    float m_top = -INFINITY;              // largest score of the row so far (ALiBi far tiles)
    float l_run = 0.0f;
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    }

    // LDS byte addresses of the lane's K operand reads in buffer 0 (row qcol, chunk
    // 2 ks + g2); rows 32.. of the tile share the swizzle of rows 0..31
    constexpr uint32_t kKBufBytes = BN * KLD * 2;
    using lds_u32x4 = const __attribute__((address_space(3))) u32x4*;
    uint32_t kaddr[KS];
#pragma unroll
    for (int ks_i = 0; ks_i < KS; ++ks_i)
        kaddr[ks_i] = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(kbuf(0))) +
                      2u * kpos(qcol, 2 * ks_i + g2);

    // ---- stage 1: S^T = K Q^T for the K tile in slot buf (plus the ALiBi term)
    auto qk = [&](int buf, f32x16 (&sacc)[2]) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.0f;
        }
        // the lane's read addresses in buffer 0 are loop-invariant (kaddr); buffer 1 is
        // one uniform add away, the second 32-key half an immediate offset
        const uint32_t boff = static_cast<uint32_t>(buf) * kKBufBytes;
#pragma unroll
        for (int ks_i = 0; ks_i < KS; ++ks_i) {
            // opaque sum, so that the second half's offset folds into the read
            uint32_t ka = kaddr[ks_i] + boff;
            asm volatile("" : "+v"(ka));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const u32x4 kop = *reinterpret_cast<lds_u32x4>(
                    static_cast<uintptr_t>(ka + mt * 32 * KLD * 2));
                sacc[mt] = mfma32x32x16<MBF>(kop, qhi[ks_i], sacc[mt]);
                if constexpr (I8) sacc[mt] = mfma32x32x16<false>(kop, qlo[ks_i], sacc[mt]);
            }
        }
        if constexpr (alibi) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) sacc[mt] = mfma32x32x8<true>(bias_a[mt], bias_b, sacc[mt]);
        }
        if constexpr (!I8) {
            // keep four operand reads in flight ahead of the MFMAs that consume them
            constexpr int NR = 2 * KS;
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);          // DS read
#pragma unroll
            for (int i = 0; i < NR - 4; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, alibi ? 6 : 4, 0);
        }
    };

    // ---- scores of one tile relative to the reference max, masked, then the row max:
    //      rows whose max exceeds the reference by more than the slack (or that see
    //      their first key) are re-based, which rescales O and l.  Afterwards every
    //      score is <= slack, so exp2 of it is safe to round to 16 bits.
    //      The key of sacc[mt][r] is j0 + 4*g2 + dj, dj = 32mt + 8(r/4) + r%4.
    //      Returns true (ALiBi, 16-bit K/V) when every score of the tile, in every row of the
    //      wave, lies more than kNegligible below the row's reference: each weight is then
    //      below 2^-32 of the reference key's, so the tile's P and P V are skipped (its
    //      share of l and O stays below 2^-32 per key, under fp32 rounding of the sums).
    auto scores = [&](f32x16 (&sacc)[2], int j0, bool need_mask, bool first) {
        const float mo = (m_ref == -INFINITY) ? 0.0f : m_ref;
        float base = -mo;
        if constexpr (alibi) base += slope2 * static_cast<float>(j0 - pos);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mt][r] = fmaf(sacc[mt][r], s_mul, base);
        }
        if (need_mask) {
            // only tiles on the causal diagonal or past kvlen; the empty asm keeps the
            // compiler from turning this wave-uniform branch into selects on every tile
            asm volatile("" ::: "memory");
            // visible keys: dj <= lim (j < kvlen, and j <= p_i when causal)
            const int lim = (causal ? min(pos, kvlen - 1) : kvlen - 1) - (j0 + 4 * g2);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int dj = 32 * mt + 8 * (r >> 2) + (r & 3);
                    sacc[mt][r] = (dj <= lim) ? sacc[mt][r] : -INFINITY;
                }
            }
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[mt][r]);
        }
        tmax = max_halves(tmax);
        if constexpr (alibi && DIRECT) m_top = fmaxf(m_top, mo + tmax);
        const bool grow = (tmax > kRescaleSlack) || (m_ref == -INFINITY && tmax > -INFINITY);
        bool negligible = false;
        if constexpr (alibi && !I8) negligible = !__any(grow || tmax >= -kNegligible);
        if (__any(grow)) {
            const float up = grow ? tmax : 0.0f;
            const float alpha = grow ? fast_exp2(m_ref - (mo + up)) : 1.0f;
            m_ref = grow ? mo + up : m_ref;
            l_run *= alpha;
            // on the wave's first tile O is still zero: nothing to rescale
            if (!first) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
            }
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) sacc[mt][r] -= up;
            }
        }
        return negligible;
    };

    // ---- P = exp2(scores), packed as the P^T operands (k-step kt holds keys
    //      16kt + 8(s/4) + 4*g2 + s%4, s = 0..7), and the row sums.  f16 P (relative
    //      rounding <= 2^-11) is summed as rounded, two values per v_dot2; bf16 rounding
    //      (2^-9) would show in lse, so bf16 sums the f32 values.
    auto probs = [&](f32x16 (&sacc)[2], u32x4 (&pop)[4]) {
        float psum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int mt = kt >> 1, rb = 8 * (kt & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p0 = fast_exp2(sacc[mt][rb + 2 * i]);
                const float p1 = fast_exp2(sacc[mt][rb + 2 * i + 1]);
                pop[kt][i] = pack2<MBF>(p0, p1);
                if constexpr (MBF) psum[i] += p0 + p1;
                else psum[i] = dot2_ones<false>(pop[kt][i], psum[i]);
            }
        }
        l_run += (psum[0] + psum[1]) + (psum[2] + psum[3]);
    };

    // ---- O^T += V^T P^T with the V tile at vs, V^T operands by transposed reads of
    //      row-major V: the first read gives keys 16kt + 4*g2 + 0..3, the second
    //      16kt + 8 + 4*g2 + 0..3
    auto pv = [&](const u32x4 (&pop)[4], const uint16_t* vs) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                // columns dt*32 + tr_col .. +3: chunk 4dt + tr_col/8, half (tr_col/4) & 1
                const int c = 4 * dt + (tr_col >> 3), h4 = 4 * ((tr_col >> 2) & 1);
                const u32x2 lo = lds_read_tr16(vs + vpos(16 * kt + tr_row, c) + h4);
                const u32x2 hi = lds_read_tr16(vs + vpos(16 * kt + 8 + tr_row, c) + h4);
                const u32x4 vop = {lo.x, lo.y, hi.x, hi.y};
                oacc[dt] = mfma32x32x16<MBF>(vop, pop[kt], oacc[dt]);
            }
        }
    };

    // Visiting order (prefill_visit): the item's last tile T, the one nearest its
    // queries, first -- under a causal mask (and even more with ALiBi, whose bias grows
    // towards the diagonal) it holds the row maxima, so later tiles rarely re-base the
    // running sums, and under ALiBi the tiles far from the queries are then recognised as
    // negligible at once; then the P tiles holding only keys before the new tokens,
    // P - 1 down to 0, which the workgroups of all query tiles of a head need and read
    // side by side on one XCD, sharing them through its L2; then the rest of the
    // diagonal.  A wave works on tiles 0 .. t_act (its rows see no key of a higher
    // tile); tiles on the diagonal or past kvlen are masked.  Step k's buffer is k % 2.
    PrefillVisit vis = prefill_visit(it.ktiles, causal, qlen, kvlen, wave_q0);
    const int T = vis.T;
    const int t_act = vis.t_act;
    auto need_mask = [&](int t) {
        return (t * BN + BN > kvlen) || (causal && t * BN + BN - 1 > wave_pmin);
    };

    auto tile_of = [&](int k) { return prefill_tile_of(vis, k); };
    int k_first = vis.k_first;
    // ALiBi over 16-bit K/V: far tiles.  Prefix tiles whose bias, at the smallest slope
    // of the workgroup's heads and the distance from its first query row to the tile's
    // last key, lies more than kFarTileBias below the nearest key's are expected to be
    // negligible for every row; they are the tiles 0 .. t_far - 1, which are bounded
    // (and, where the bound holds, skipped) after the other tiles are computed.
    float wg_slope2 = 0.0f;
    if constexpr (alibi && DIRECT) {
        wg_slope2 = INFINITY;
        for (int i = 0; i < heads; ++i) wg_slope2 = fminf(wg_slope2, a.slopes[it.h + i] * kLog2e);
    }
    const int wg_pmin = shift + it.qbeg;
    auto far = [&](int t) {
        return t < vis.P && wg_slope2 * static_cast<float>(wg_pmin - (t * BN + BN - 1)) > kFarTileBias;
    };
    auto compute = [&](int t, int buf, bool first) {
        if (t <= t_act) {
            f32x16 sacc[2];
            u32x4 pop[4];
            qk(buf, sacc);
            if (!scores(sacc, t * BN, need_mask(t), first)) {
                probs(sacc, pop);
                pv(pop, vbuf(buf));
            }
        }
    };
    // plain double-buffered steps k0 .. k1 - 1: tile k in K slot k % 2 and V slot 2 + k % 2;
    // the loads into slot (k+1) % 2 start after the barrier that follows every read of its
    // previous tile (step k - 1); vmcnt(0) + barrier publish them
    auto plain_steps = [&](int k0, int k1) {
        if (k0 < k1) load_tile_direct(k0 & 1, tile_of(k0), true, true);
        for (int k = k0; k < k1; ++k) {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            __syncthreads();
            if (k + 1 < k1) load_tile_direct((k + 1) & 1, tile_of(k + 1), true, true);
            compute(tile_of(k), k & 1, k == k_first);
        }
    };
    if constexpr (DIRECT && alibi) {
        int t_far = 0;                  // far(t) holds for t < t_far (it falls with t)
        if (wg_slope2 > 0.0f)
            while (t_far < vis.P && far(t_far)) ++t_far;
        t_far = __builtin_amdgcn_readfirstlane(t_far);      // the same in every lane
        if (t_far == 0) {
            plain_steps(0, T + 1);
        } else {
            // the near tiles first, T down to t_far (the diagonal, then the prefix tiles
            // near enough to matter), double-buffered as in plain_steps, so that every row
            // holds its reference from its nearest keys; the far tiles (t_far - 1 ..
            // 0) last
            const int n_near = T - t_far + 1;
            vis.P = 0;                  // the plain visit order is then T, T - 1, ...
            k_first = (t_act >= t_far) ? T - t_act : n_near;        // first tile it sees
            plain_steps(0, n_near);
            // the smallest row maximum among the workgroup's query rows
            {
                const float mm = wave_min(qvalid ? m_top : INFINITY);
                if (lane == 0) s_mmin[wave] = mm;
            }
            __syncthreads();            // every wave is done with the last plain tile
            const float mmin = fminf(fminf(s_mmin[0], s_mmin[1]), fminf(s_mmin[2], s_mmin[3]));
            // The far tiles in two passes.  Pass A: every wave streams its own 16 K rows of
            // each far tile into registers (no LDS, no barrier) and bounds the tile's
            // scores against those rows (Cauchy-Schwarz: |s_mul q . k| <= max |s_mul q| *
            // |k|, plus the tile's largest bias).  A tile whose bound lies below every
            // row's largest score so far by more than kNegligible + 1 (the 1 for rounding)
            // adds weights under 2^-33 of a row's largest, which l already holds, and
            // re-bases no row: it is skipped.  The bound holds for the tile when it holds
            // for each wave's rows, so a wave keeps only the first and the last far tile
            // its rows leave uncovered.  Pass B: after one barrier, the tiles from the
            // first to the last uncovered one of any wave are computed as plain tiles.
            const int F = t_far;
            const float qmax = fmaxf(fmaxf(s_qmax[0], s_qmax[1]), fmaxf(s_qmax[2], s_qmax[3]));
            const float thr = mmin - kNegligible - 1.0f;
            using gu32x4 = const __attribute__((address_space(1))) u32x4;
            // the wave's rows of far tile f, load i covering row RPI*i + lrow (chunks in
            // the swizzled order of the LDS loads: a permutation inside each row); the
            // uniform base and the lane's 32-bit offset give the scalar-base load form
            auto far_load = [&](u32x4 (&x)[NL], int f) {
                const int g0 = (t_far - 1 - f) * BN + 16 * wave;
                const int blk = bshift >= 0 ? (g0 >> bshift)
                                            : static_cast<int>(static_cast<uint32_t>(g0) / static_cast<uint32_t>(bs));
                const uint32_t slotoff = static_cast<uint32_t>(g0 - blk * bs);
                const uint64_t e = static_cast<uint32_t>(ctab[blk]);
                uint64_t bi = reinterpret_cast<uintptr_t>(kpool + e * static_cast<uint64_t>(kblk_bytes) + slotoff * kslot32);
                asm volatile("" : "+s"(bi));
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    uint32_t o = koff_full[i];
                    asm volatile("" : "+v"(o));
                    x[i] = *reinterpret_cast<gu32x4*>(bi + o);
                }
            };
            // tile f's bound against the wave's rows.  For load i the lane holds P_i, the
            // sum of squares of its 8 elements of row RPI*i + lrow; a row's |k|^2 is the
            // sum of its P over the CH lanes of its group, so the largest |k|^2 among the
            // group's rows is at most the group's sum of each lane's largest P_i (one
            // reduction per tile rather than one per row; NaN propagates).  The bound holds
            // iff qmax^2 * that < c^2 with c = thr - the tile's largest bias > 0.
            const float qmax2 = qmax * qmax;
            int f_lo = F, f_hi = -1;                // the wave's first / last uncovered tile
            auto check = [&](const u32x4 (&x)[NL], int f) {
                float pm = 0.0f;
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    float ss = 0.0f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) ss = dot2_self<MBF>(x[i][e], ss);
                    pm = __builtin_elementwise_maximum(pm, ss);
                }
                const float g = group_sum<CH>(pm);
                const int t = t_far - 1 - f;
                const float c = thr - wg_slope2 * static_cast<float>(t * BN + BN - 1 - wg_pmin);
                const bool ok = c > 0.0f && g * qmax2 < c * c;
                if (__any(!ok)) {
                    f_lo = f_lo < f ? f_lo : f;
                    f_hi = f;
                }
            };
            // kDepth tiles in flight; the loads are unconditional (an index past the run
            // re-reads its last tile), which keeps the compiler's waits exact
            constexpr int kDepth = 4;
            u32x4 xb[kDepth][NL];
#pragma unroll
            for (int d = 0; d < kDepth; ++d) far_load(xb[d], d < F ? d : F - 1);
            int f0 = 0;
            for (; f0 + kDepth < F; f0 += kDepth) {
#pragma unroll
                for (int d = 0; d < kDepth; ++d) {
                    check(xb[d], f0 + d);
                    const int fn = f0 + d + kDepth;
                    far_load(xb[d], fn < F ? fn : F - 1);
                }
            }
#pragma unroll
            for (int d = 0; d < kDepth; ++d)
                if (f0 + d < F) check(xb[d], f0 + d);
            if (lane == 0) {
                s_frange[0][wave] = f_lo;
                s_frange[1][wave] = f_hi;
            }
            __syncthreads();
            const int lo = __builtin_amdgcn_readfirstlane(
                min(min(s_frange[0][0], s_frange[0][1]), min(s_frange[0][2], s_frange[0][3])));
            const int hi = __builtin_amdgcn_readfirstlane(
                max(max(s_frange[1][0], s_frange[1][1]), max(s_frange[1][2], s_frange[1][3])));
            if (lo <= hi) {
                // Pass B (plain step k visits tile T - k); the barrier frees the buffers
                // for the epilogue
                plain_steps(n_near + lo, n_near + hi + 1);
                __syncthreads();
            }
        }
    } else if constexpr (DIRECT) {
        plain_steps(0, T + 1);
    } else {
        if (T >= 0) {
            load_k(tile_of(0));
            load_v(tile_of(0));
        }
        for (int k = 0; k <= T; ++k) {
            const int t = tile_of(k);
            store_k(k & 1);
            store_v(k & 1, t);
            __syncthreads();
            if (k < T) {
                load_k(tile_of(k + 1));
                load_v(tile_of(k + 1));
            }
            compute(t, k & 1, k == k_first);
        }
    }

    // ------------------------------------------------------------- epilogue
    // O = O^T / l, rounded to the output type, goes through LDS so that the global
    // stores write whole rows: a lane holds 4-element pieces of one query row, and
    // storing those directly leaves 32 rows half-written per instruction.  Each wave
    // stages its 32 x D tile in its own quarter of the K/V buffer pair that no wave reads
    // any more (buffer (T + 1) % 2: its last tile was consumed before the last barrier
    // and nothing is loaded into it afterwards), 16-byte chunks of row r placed at chunk
    // c ^ (r % NCH) so that both the 8-byte writes and the 16-byte reads are free of
    // bank conflicts.
    const float L = sum_halves(l_run);
    const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
    constexpr int NCH = D / 8;                  // 16-byte chunks per output row
    uint16_t* stage = ((wave < 2) ? kbuf((T + 1) & 1) : vbuf((T + 1) & 1)) + (wave & 1) * (32 * D);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const int d0 = dt * 32 + 8 * r4 + 4 * g2;     // rows 4 consecutive d
            float o[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float val = oacc[dt][4 * r4 + c] * inv;
                if constexpr (I8) {
                    if (!vtok) {
                        const bool f32 = a.aq.extended ? a.aq.vscale_is_f32 != 0 : a.scale_is_f32 != 0;
                        auto chan = [&](const void* src) {
                            return f32 ? static_cast<const float*>(src)[kvh_off + d0 + c]
                                       : half_to_f32<BF16>(static_cast<const uint16_t*>(src)[kvh_off + d0 + c]);
                        };
                        if (a.aq.voff != nullptr && L > 0.0f) val += chan(a.aq.voff);
                        val *= chan(a.vscale);
                    }
                }
                o[c] = val;
            }
            u32x2 w;
            w.x = pack2<BF16>(o[0], o[1]);
            w.y = pack2<BF16>(o[2], o[3]);
            const int chunk = (dt * 4 + r4) ^ (qcol % NCH);
            *reinterpret_cast<u32x2*>(stage + qcol * D + chunk * 8 + 4 * g2) = w;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {
        constexpr int RPI = 64 / NCH;           // rows per store instruction
        const int c = lane % NCH;
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
            const int r = i * RPI + lane / NCH;
            const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * D + (c ^ (r % NCH)) * 8);
            if (wave_q0 + r < qlen) {
                uint16_t* orow = static_cast<uint16_t*>(a.out) +
                                 static_cast<int64_t>(it.qrow0 + wave_q0 + r) * a.out_tok_stride +
                                 static_cast<int64_t>(h) * a.out_head_stride;
                *reinterpret_cast<u32x4*>(orow + 8 * c) = x;
            }
        }
    }
    if (!qvalid) return;
    if (g2 == 0 && a.lse != nullptr) {
        a.lse[static_cast<int64_t>(it.qrow0 + qi) * a.lse_tok_stride + h] =
            (L > 0.0f) ? (m_ref + kconst + fast_log2(L)) * kLn2 : INFINITY;
    }
}

template <int D, bool BF16, bool I8, bool F8>
hipError_t launch_prefill_t(const PrefillArgs& a, int n_items, hipStream_t stream, hipEvent_t t0,
                            hipEvent_t t1) {
    if (a.mask_type == PA_MASK_ALIBI)
        launch_256(prefill_kernel<D, BF16, I8, F8, 2>, n_items, stream, t0, t1, a);
    else if (a.mask_type == PA_MASK_CAUSAL)
        launch_256(prefill_kernel<D, BF16, I8, F8, 1>, n_items, stream, t0, t1, a);
    else
        launch_256(prefill_kernel<D, BF16, I8, F8, 0>, n_items, stream, t0, t1, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_d(const PrefillArgs& a, int n_items, bool bf16, bool i8, bool f8,
                            hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    if (f8) return bf16 ? launch_prefill_t<D, true, true, true>(a, n_items, stream, t0, t1)
                        : launch_prefill_t<D, false, true, true>(a, n_items, stream, t0, t1);
    if (i8) return bf16 ? launch_prefill_t<D, true, true, false>(a, n_items, stream, t0, t1)
                        : launch_prefill_t<D, false, true, false>(a, n_items, stream, t0, t1);
    return bf16 ? launch_prefill_t<D, true, false, false>(a, n_items, stream, t0, t1)
                : launch_prefill_t<D, false, false, false>(a, n_items, stream, t0, t1);
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int n_items, int head_size, bool bf16, bool i8,
                          bool f8, hipStream_t stream, hipEvent_t t0, hipEvent_t t1) {
    if (n_items <= 0) return hipSuccess;
    if (head_size == 128) return launch_prefill_d<128>(a, n_items, bf16, i8, f8, stream, t0, t1);
    return launch_prefill_d<64>(a, n_items, bf16, i8, f8, stream, t0, t1);
}

}  // namespace pa
