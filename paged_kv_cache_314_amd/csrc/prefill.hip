// Paged prefill / prefix-encoder attention on gfx950 (seqLen > 1 queries per sequence).
//
// Operation: aclnnFusedInferAttentionScoreV4, "Function" (softmax(scale*QK^T + mask) V),
// prefill scenario; PrefixEncoder (Definition, Members): the new query tokens of a
// sequence attend over its paged cache of kvSeqLen tokens (cached prefix + new tokens),
// maskType 9 = causal mask generated internally, maskType 3 = ALiBi bias
// slopes[h] * (j - p_i) plus causal, qkScale post-multiplying Q*K^T.  Query i of a
// sequence sits at absolute position p_i = kvSeqLen - seqLen + i.
//
// One workgroup = 4 waves = 128 query rows of one (sequence, head); wave w owns rows
// 32w .. 32w+31.  Keys are visited in tiles of 64 up to the last key any of the 128 rows
// can see.  Per tile:
//   all threads: K tile (64 x D) -> LDS row-major; V tile -> LDS transposed (V^T, keys
//                permuted so each lane's 8 MFMA k-slots are 16 contiguous bytes)
//   per wave:    S^T[64 keys x 32 rows] = K . Q^T      (D/16 x 2 MFMA 32x32x16)
//                scale, ALiBi bias, causal / tail mask, online softmax, in registers:
//                a lane owns one query row, so row max / sum need one cross-lane step
//                O^T[D x 32 rows] += V^T . P^T          (D/32 x 4 MFMA 32x32x16)
// Q stays in registers as the B operand; LDS is double-buffered so one barrier per key
// tile suffices, and the next tile's global loads are in flight during the MFMA work.
// int8 K/V are converted exactly to f16 on the way into LDS; the per-channel K scale is
// folded into Q (kept to ~22 bits as an f16 hi + lo pair), the V scale into the output.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_kernels.h"

namespace pa {

namespace {

constexpr int BM = kPrefillBM;   // 128 query rows per workgroup
constexpr int BN = kPrefillBN;   // 64 keys per tile
constexpr int KPAD = 8;          // LDS row padding (16-bit elements) against bank conflicts
constexpr int VPAD = 8;

// LDS position of key tau (0..63) inside a V^T row: tau = 16*kt + 8*a + 4*g + c is
// placed at 16*kt + 8*g + 4*a + c, so lane group g reads keys {16kt + 4g + 0..3,
// 16kt + 8 + 4g + 0..3} as one 16-byte run -- the k-slot order of the P^T operand.
__device__ __forceinline__ int vt_pos4(int tg4) {   // position of key 4*tg4 (c = 0)
    return 16 * (tg4 >> 2) + 8 * (tg4 & 1) + 4 * ((tg4 >> 1) & 1);
}

template <int D, bool BF16, bool I8>
__global__ void __launch_bounds__(256, 2) prefill_kernel(PrefillArgs a) {
    constexpr bool MBF = BF16 && !I8;
    constexpr int KS = D / 16;            // QK k-steps (32x32x16)
    constexpr int DT = D / 32;            // PV output row blocks
    constexpr int KLD = D + KPAD;         // K tile LDS row length
    constexpr int VLD = BN + VPAD;        // V^T LDS row length
    // 16-bit global K loads: D/8 chunks of 16 bytes per key row
    constexpr int CH = D / 8;
    constexpr int NK = I8 ? (BN * (D / 16) + 255) / 256 : (BN * CH + 255) / 256;
    constexpr int NV = (16 * CH + 255) / 256;   // V sub-blocks (4 keys x 8 d) per thread

    __shared__ uint16_t s_k[2][BN * KLD];
    __shared__ uint16_t s_v[2][D * VLD];

    const PrefillItem it = a.items[blockIdx.x];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qcol = lane & 31;           // query row of this lane inside the wave
    const int g2 = lane >> 5;             // k-slot half
    const int kvh = it.h / a.group;
    const int64_t kvh_off = static_cast<int64_t>(kvh) * D;      // into the [Hkv, D] scales
    const int64_t k_head_off = static_cast<int64_t>(kvh) * a.k_head_stride;
    const int64_t v_head_off = static_cast<int64_t>(kvh) * a.v_head_stride;
    const int kvlen = it.kvlen;
    const int qlen = it.qlen;
    const bool causal = a.mask_type == PA_MASK_CAUSAL || a.mask_type == PA_MASK_ALIBI;
    const int shift = kvlen - qlen;       // p_i = shift + i

    const int qi = it.qbeg + 32 * wave + qcol;            // local query row of this lane
    const bool qvalid = qi < qlen;
    const int pos = shift + qi;                           // its absolute position
    const int wave_q0 = it.qbeg + 32 * wave;
    const int wave_q1 = min(wave_q0 + 31, qlen - 1);      // last valid row of the wave
    const bool wave_live = wave_q0 < qlen;
    const int wave_pmin = shift + wave_q0;
    const int wave_pmax = shift + wave_q1;

    // ---------------------------------------------------------------- Q^T
    u32x4 qhi[KS], qlo[KS];
    float s_mul;
    {
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               static_cast<int64_t>(it.qrow0 + (qvalid ? qi : 0)) * a.q_tok_stride +
                               static_cast<int64_t>(it.h) * a.q_head_stride;
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
                    float sk;
                    if (a.scale_is_f32) sk = static_cast<const float*>(a.kscale)[kvh_off + d0 + e];
                    else sk = half_to_f32<BF16>(static_cast<const uint16_t*>(a.kscale)[kvh_off + d0 + e]);
                    qf[ks][e] = qv * sk * a.scale_log2;
                    amax = fmaxf(amax, fabsf(qf[ks][e]));
                }
            }
            amax = fmaxf(amax, shfl_xor_f(amax, 32));
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
    const float slope2 = (a.mask_type == PA_MASK_ALIBI) ? a.slopes[it.h] * kLog2e : 0.0f;

    // ---------------------------------------------------------- tile loads
    const int32_t* trow = a.table + static_cast<int64_t>(it.b) * a.table_stride;
    const int bs = a.block_size;
    const float inv_bs = 1.0f / static_cast<float>(bs);
    const bool one_block_per_tile = (bs % BN) == 0;

    // element offset of key j0 + delta (j0 = first key of the tile, delta < 64)
    auto key_off = [&](int j0, int delta, int phys0, int r0, int64_t blk_stride,
                       int64_t slot_stride, int64_t head_off) -> int64_t {
        if (one_block_per_tile) {
            return static_cast<int64_t>(phys0) * blk_stride +
                   static_cast<int64_t>(r0 + delta) * slot_stride + head_off;
        }
        const int u = r0 + delta;
        const int nb = static_cast<int>((static_cast<float>(u) + 0.5f) * inv_bs);
        const int phys = trow[j0 / bs + nb];
        return static_cast<int64_t>(phys) * blk_stride +
               static_cast<int64_t>(u - nb * bs) * slot_stride + head_off;
    };

    u32x4 kreg[NK];
    u32x4 vreg[NV][4];
    auto load_tile = [&](int jt) {
        const int j0 = jt * BN;
        const int blk = j0 / bs;
        const int r0 = j0 - blk * bs;
        const int phys0 = one_block_per_tile ? trow[blk] : 0;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int idx = i * 256 + tid;
            u32x4 z = {0u, 0u, 0u, 0u};
            if constexpr (!I8) {
                const int delta = idx / CH, chunk = idx % CH;
                const bool ok = (idx < BN * CH) && (j0 + delta < kvlen);
                if (ok) {
                    const uint16_t* p = static_cast<const uint16_t*>(a.k) +
                                        key_off(j0, delta, phys0, r0, a.k_blk_stride, a.k_slot_stride, k_head_off);
                    kreg[i] = *reinterpret_cast<const u32x4*>(p + 8 * chunk);
                } else {
                    kreg[i] = z;
                }
            } else {
                constexpr int CH16 = D / 16;
                const int delta = idx / CH16, chunk = idx % CH16;
                const bool ok = (idx < BN * CH16) && (j0 + delta < kvlen);
                if (ok) {
                    const int8_t* p = static_cast<const int8_t*>(a.k) +
                                      key_off(j0, delta, phys0, r0, a.k_blk_stride, a.k_slot_stride, k_head_off);
                    kreg[i] = *reinterpret_cast<const u32x4*>(p + 16 * chunk);
                } else {
                    kreg[i] = z;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int sb = i * 256 + tid;            // sub-block: keys 4*tg4.., d 8*dg..
            const int dg = sb % CH, tg4 = sb / CH;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int delta = 4 * tg4 + c;
                const bool ok = (sb < 16 * CH) && (j0 + delta < kvlen);
                u32x4 z = {0u, 0u, 0u, 0u};
                if (!ok) {
                    vreg[i][c] = z;
                    continue;
                }
                const int64_t off = key_off(j0, delta, phys0, r0, a.v_blk_stride, a.v_slot_stride, v_head_off);
                if constexpr (!I8) {
                    vreg[i][c] = *reinterpret_cast<const u32x4*>(
                        static_cast<const uint16_t*>(a.v) + off + 8 * dg);
                } else {
                    const u32x2 raw = *reinterpret_cast<const u32x2*>(
                        static_cast<const int8_t*>(a.v) + off + 8 * dg);
                    const u32x2 c0 = i8x4_to_f16x4(raw.x), c1 = i8x4_to_f16x4(raw.y);
                    vreg[i][c] = u32x4{c0.x, c0.y, c1.x, c1.y};
                }
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t* ks = s_k[buf];
        uint16_t* vs = s_v[buf];
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int idx = i * 256 + tid;
            if constexpr (!I8) {
                if (idx < BN * CH) {
                    const int delta = idx / CH, chunk = idx % CH;
                    *reinterpret_cast<u32x4*>(ks + delta * KLD + 8 * chunk) = kreg[i];
                }
            } else {
                constexpr int CH16 = D / 16;
                if (idx < BN * CH16) {
                    const int delta = idx / CH16, chunk = idx % CH16;
                    const u32x2 c0 = i8x4_to_f16x4(kreg[i].x), c1 = i8x4_to_f16x4(kreg[i].y);
                    const u32x2 c2 = i8x4_to_f16x4(kreg[i].z), c3 = i8x4_to_f16x4(kreg[i].w);
                    uint16_t* dst = ks + delta * KLD + 16 * chunk;
                    *reinterpret_cast<u32x4*>(dst) = u32x4{c0.x, c0.y, c1.x, c1.y};
                    *reinterpret_cast<u32x4*>(dst + 8) = u32x4{c2.x, c2.y, c3.x, c3.y};
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int sb = i * 256 + tid;
            if (sb < 16 * CH) {
                const int dg = sb % CH, tg4 = sb / CH;
                const int p0 = vt_pos4(tg4);
#pragma unroll
                for (int n = 0; n < 8; ++n) {
                    const uint32_t w0 = vreg[i][0][n >> 1], w1 = vreg[i][1][n >> 1];
                    const uint32_t w2 = vreg[i][2][n >> 1], w3 = vreg[i][3][n >> 1];
                    u32x2 t;
                    t.x = (n & 1) ? pack_hi(w0, w1) : pack_lo(w0, w1);
                    t.y = (n & 1) ? pack_hi(w2, w3) : pack_lo(w2, w3);
                    *reinterpret_cast<u32x2*>(vs + (8 * dg + n) * VLD + p0) = t;
                }
            }
        }
    };

    // --------------------------------------------------------------- state
    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.0f;
    }

    const int ktiles = it.ktiles;
    if (ktiles > 0) load_tile(0);
    for (int jt = 0; jt < ktiles; ++jt) {
        const int buf = jt & 1;
        store_tile(buf);
        __syncthreads();
        if (jt + 1 < ktiles) load_tile(jt + 1);

        const int j0 = jt * BN;
        // skip the MFMA work when no row of this wave sees any key of the tile
        const bool active = wave_live && (!causal || j0 <= wave_pmax);
        if (!active) continue;
        const bool need_mask = (j0 + BN > kvlen) || (causal && j0 + BN - 1 > wave_pmin);

        // ---- S^T = K Q^T
        f32x16 sacc[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[mt][r] = 0.0f;
        }
        const uint16_t* ks = s_k[buf];
#pragma unroll
        for (int ks_i = 0; ks_i < KS; ++ks_i) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const u32x4 kop = *reinterpret_cast<const u32x4*>(
                    ks + (mt * 32 + qcol) * KLD + 16 * ks_i + 8 * g2);
                sacc[mt] = mfma32x32x16<MBF>(kop, qhi[ks_i], sacc[mt]);
                if constexpr (I8) sacc[mt] = mfma32x32x16<false>(kop, qlo[ks_i], sacc[mt]);
            }
        }
        // ---- scale, bias, mask; key of sacc[mt][r] = j0 + 32mt + 8(r/4) + 4*g2 + r%4
        const float bias0 = slope2 * static_cast<float>(j0 + 4 * g2 - pos);
        float tmax = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dj = 32 * mt + 8 * (r >> 2) + (r & 3);
                float x = sacc[mt][r] * s_mul;
                if (a.mask_type == PA_MASK_ALIBI) x += bias0 + slope2 * static_cast<float>(dj);
                if (need_mask) {
                    const int j = j0 + 4 * g2 + dj;
                    const bool vis = (j < kvlen) && (!causal || j <= pos);
                    x = vis ? x : -INFINITY;
                }
                sacc[mt][r] = x;
                tmax = fmaxf(tmax, x);
            }
        }
        tmax = fmaxf(tmax, shfl_xor_f(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float psum = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = fast_exp2(sacc[mt][r] - m_use);
                sacc[mt][r] = p;
                psum += p;
            }
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;

        // ---- P^T operands: k-step kt holds keys 16kt + 8(s/4) + 4*g2 + s%4, s = 0..7
        u32x4 pop[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            const int mt = kt >> 1, rb = 8 * (kt & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                pop[kt][i] = pack2<MBF>(sacc[mt][rb + 2 * i], sacc[mt][rb + 2 * i + 1]);
        }
        // ---- O^T += V^T P^T
        const uint16_t* vs = s_v[buf];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                const u32x4 vop = *reinterpret_cast<const u32x4*>(
                    vs + (dt * 32 + qcol) * VLD + 16 * kt + 8 * g2);
                oacc[dt] = mfma32x32x16<MBF>(vop, pop[kt], oacc[dt]);
            }
        }
    }

    // ------------------------------------------------------------- epilogue
    const float L = l_run + shfl_xor_f(l_run, 32);
    if (!qvalid) return;
    const float inv = (L > 0.0f) ? 1.0f / L : 0.0f;
    uint16_t* orow = static_cast<uint16_t*>(a.out) +
                     static_cast<int64_t>(it.qrow0 + qi) * a.out_tok_stride +
                     static_cast<int64_t>(it.h) * a.out_head_stride;
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
                    float sv;
                    if (a.scale_is_f32) sv = static_cast<const float*>(a.vscale)[kvh_off + d0 + c];
                    else sv = half_to_f32<BF16>(static_cast<const uint16_t*>(a.vscale)[kvh_off + d0 + c]);
                    val *= sv;
                }
                o[c] = val;
            }
            u32x2 w;
            w.x = pack2<BF16>(o[0], o[1]);
            w.y = pack2<BF16>(o[2], o[3]);
            *reinterpret_cast<u32x2*>(orow + d0) = w;
        }
    }
    if (g2 == 0 && a.lse != nullptr) {
        a.lse[static_cast<int64_t>(it.qrow0 + qi) * a.lse_tok_stride + it.h] =
            (L > 0.0f) ? (m_run + fast_log2(L)) * kLn2 : INFINITY;
    }
}

template <int D, bool BF16, bool I8>
hipError_t launch_prefill_t(const PrefillArgs& a, int n_items, hipStream_t stream) {
    hipLaunchKernelGGL((prefill_kernel<D, BF16, I8>), dim3(n_items), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, int n_items, int head_size, bool bf16, bool i8,
                          hipStream_t stream) {
    if (n_items <= 0) return hipSuccess;
    if (head_size == 128) {
        if (i8) return bf16 ? launch_prefill_t<128, true, true>(a, n_items, stream)
                            : launch_prefill_t<128, false, true>(a, n_items, stream);
        return bf16 ? launch_prefill_t<128, true, false>(a, n_items, stream)
                    : launch_prefill_t<128, false, false>(a, n_items, stream);
    }
    if (i8) return bf16 ? launch_prefill_t<64, true, true>(a, n_items, stream)
                        : launch_prefill_t<64, false, true>(a, n_items, stream);
    return bf16 ? launch_prefill_t<64, true, false>(a, n_items, stream)
                : launch_prefill_t<64, false, false>(a, n_items, stream);
}

}  // namespace pa
