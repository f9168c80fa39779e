// Chunked KDA forward on gfx950 MFMA (bf16 operands, fp32 state), dk = dv = 128.
//
// The recurrence is Eq. 14 of Chimera page 1, section 3.3 (parentheses as on
// page 2): S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T, read out
// as o_t = S_t^T q_t (Eq. 15, inner term). The pages give no chunked form; the
// one used here follows from Eq. 14 by unrolling it over a chunk of 64 tokens.
// With g_r = sum_{i<=r} log a_i per key channel (restarting every chunk),
// incoming state S and u_r = b_r (v_r - S_{r-1}^T Diag(a_r) k_r):
//
//   S_r = Diag(e^{g_r}) (S + sum_{i<=r} (k_i e^{-g_i}) u_i^T)
//   (I + A) U = diag(b) V - diag(b) (K e^g) S,  A_ri = b_r sum_c k_rc k_ic e^{g_rc - g_ic}  (i < r)
//   O = (Q e^g) S + Aqk U,                      Aqk_ri = sum_c q_rc k_ic e^{g_rc - g_ic}  (i <= r)
//   S_next = Diag(e^{g_n}) S + (K e^{g_n - g})^T U
//
// so with T = (I + A)^{-1}, W = T diag(b) K e^g and U~ = T diag(b) V, the chunk
// step is U = U~ - W S. The pairwise factors e^{g_r - g_i} are split around a
// reference token in the middle of each 16-token block, so every factored
// operand stays within the decay of 8 tokens. Decays are formed as running
// products of alpha (no log / exp). The per-(token, head) L2 normalisation of
// q and k (page 1, Fig. 2) is applied as row/column scalings of A, Aqk, W, U
// and O rather than to the operands.
//
// The sequence is cut into P segments of L chunks per (batch, head) so that the
// chip has enough independent work:
//   pass 1 (summary):  each segment runs the recurrence on [S | M] from [0 | I],
//                      giving S_p (zero start) and the transition M_p;
//   pass 2 (combine):  S_start(p+1) = M_p S_start(p) + S_p, fp32 MFMA;
//   pass 3 (output):   each segment reruns from S_start(p), writing o.
// With P = 1 only pass 3 runs, starting from S0.
#include "dtypes.h"
#include "internal.h"

namespace chm {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));

constexpr int D = 128;      // dk = dv
constexpr int CT = 64;      // tokens per chunk
constexpr int SBT = 16;     // tokens per decay block
constexpr int NSB = CT / SBT;
constexpr int NTHR = 512;   // 8 waves
constexpr float kL2Eps = 1e-6f;
constexpr int kTargetBlocks = 256;   // one block per CU

__device__ __forceinline__ f32x4 mma32(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b), c,
                                                   0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint2 pack4(const f32x4& v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ uint4 pack8(const f32x4& lo, const f32x4& hi) {
  return make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(hi[0], hi[1]),
                    pack_bf16x2(hi[2], hi[3]));
}
__device__ __forceinline__ uint4 cat(uint2 a, uint2 b) { return make_uint4(a.x, a.y, b.x, b.y); }

// index of the (I, J) block pair with I > J
__device__ __forceinline__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }

// LDS arrays are flat with padded rows so that the MFMA operand reads (16
// consecutive rows, same column) and the elementwise writes hit distinct banks;
// the padding is additive, so every address folds into an instruction offset.
//   rm: [CT][D] row-major, row stride D + 8 elements (272 bytes)
//   tr: [D][CT] and [CT][CT], row stride CT + 4 elements (136 bytes)
constexpr int RMS = D + 8;
constexpr int TRS = CT + 4;
__device__ __forceinline__ int rm(int row, int col) { return row * RMS + col; }
__device__ __forceinline__ int tr(int row, int col) { return row * TRS + col; }

struct Lds {
  uint16_t kr[CT * RMS];  // rm: k e^{g - m_I}        row operand of A;   then -W ([token][dk])
  uint16_t kc[CT * RMS];  // rm: k e^{m_I - g}        column operand of A and Aqk
  uint16_t qr[CT * RMS];  // rm: q e^{g - m_I}        row operand of Aqk; then the output tile
  uint16_t qh[CT * RMS];  // rm: q e^{g}              operand of Q^ S
  uint16_t kbT[D * TRS];  // tr: (k e^{g})^T          right-hand side of W
  uint16_t vT[D * TRS];   // tr: v^T                  right-hand side of U~
  uint16_t ktT[D * TRS];  // tr: (k e^{g_n - g})^T    operand of the state update
  uint16_t at[CT * TRS];  // tr: -A in blocks below the diagonal, T_II on the diagonal blocks
  uint16_t aqk[CT * TRS]; // tr: Aqk, row i scaled by 1/|q_i|, column j by 1/|k_j|
  float adiag[NSB][SBT][20];   // strictly lower A_II, column k stored at 4*(k&3) + (k>>2)
  float pb[NSB][D];       // per block and channel: product of alpha over block tokens 0..8
  float pf[NSB][D];       //                        ... over block tokens 9..15
  float pij[6][D];        // e^{m_I - m_J}, I > J
  float egn[D];           // e^{g_n}
  float beta[CT];
  float rk[CT];           // 1/|k_t| (1 without normalisation)
  float rq[CT];
};

struct ChunkArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int64_t stride;
  const uint16_t* alpha;
  const uint16_t* beta;
  const float* S0;        // output pass without split: [BH][D][D] or null
  const float* Sstart;    // output pass with split: [BH][P][D][D]
  float* SM;              // summary pass: [BH][P][D][2D]
  uint16_t* o;
  float* S_final;
  int64_t T;
  int64_t H;
  int P;                  // segments per (batch, head)
  int L;                  // chunks per segment
  int l2norm;
};

// Register-level lane exchanges (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_xor1(float v) { return dpp_f<0xB1>(v); }              // quad_perm 1,0,3,2
__device__ __forceinline__ float lane_xor2(float v) { return dpp_f<0x4E>(v); }              // quad_perm 2,3,0,1
__device__ __forceinline__ float lane_xor4(float v) { return dpp_f<0x1B>(dpp_f<0x141>(v)); } // half mirror, quad reverse
__device__ __forceinline__ float lane_xor8(float v) { return dpp_f<0x128>(v); }             // row_ror 8
// a + (the partner's b) with partner = lane ^ 32 (lanes < 32 get lo + lo', lanes >= 32 get hi' + hi)
__device__ __forceinline__ float halve32(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(lo), __float_as_int(hi), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}
// the same across 16-lane rows: lanes with bit 4 clear get lo + lo', set get hi' + hi
__device__ __forceinline__ float halve16(float lo, float hi) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(lo), __float_as_int(hi), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// Sum 16 per-lane values over the 64 lanes of a wave by recursive halving.
// Returns the total of value v in the lanes with (lane & 3) == 0, where
// v = bit2 + 2*bit3 + 4*bit4 + 8*bit5 of the lane id.
__device__ __forceinline__ float wave_sum16(const float (&a)[16], int lane) {
  float b8[8], b4[4], b2[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) b8[j] = halve32(a[j], a[j + 8]);
#pragma unroll
  for (int j = 0; j < 4; ++j) b4[j] = halve16(b8[j], b8[j + 4]);
  const bool u3 = (lane >> 3) & 1, u2 = (lane >> 2) & 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) b2[j] = (u3 ? b4[j + 2] : b4[j]) + lane_xor8(u3 ? b4[j] : b4[j + 2]);
  float b1 = (u2 ? b2[1] : b2[0]) + lane_xor4(u2 ? b2[0] : b2[1]);
  b1 += lane_xor2(b1);
  b1 += lane_xor1(b1);
  return b1;
}

__device__ __forceinline__ uint4 ld128(const uint16_t* base, int idx) {
  return *reinterpret_cast<const uint4*>(base + idx);
}
// MFMA fragment with the K order permuted as 32s + 4q + (0..3), 32s + 16 + 4q + (0..3)
__device__ __forceinline__ uint4 ld_perm(const uint16_t* base, int row_idx, int k0) {
  return cat(*reinterpret_cast<const uint2*>(base + row_idx + k0), *reinterpret_cast<const uint2*>(base + row_idx + k0 + 16));
}

// Raw inputs of one chunk for one lane: tokens tk0..tk0+7 of the chunk,
// channels ch, ch+1 (packed bf16 pairs).
struct ChunkRegs {
  uint32_t k[8], v[8], q[8], al[8];
  uint32_t a8;   // alpha of the block's token 8 (lower half only)
};

template <bool OUT>
__device__ __forceinline__ void load_chunk(const ChunkArgs& a, int64_t b, int64_t h, int64_t t0, int n, int tk0,
                                           bool lower_half, int ch, ChunkRegs& R) {
  const int64_t row = b * a.T + t0 + tk0;
  const uint32_t* kp = reinterpret_cast<const uint32_t*>(a.k + row * a.stride + h * D + ch);
  const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.v + row * a.stride + h * D + ch);
  const uint32_t* qp = reinterpret_cast<const uint32_t*>(a.q + row * a.stride + h * D + ch);
  const uint32_t* ap = reinterpret_cast<const uint32_t*>(a.alpha + (row * a.H + h) * D + ch);
  const int64_t st = a.stride / 2, sa = a.H * D / 2;   // token strides in 32-bit words
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (tk0 + i < n) {
      R.k[i] = kp[i * st];
      R.v[i] = vp[i * st];
      R.q[i] = OUT ? qp[i * st] : 0u;
      R.al[i] = ap[i * sa];
    } else {
      R.k[i] = R.v[i] = R.q[i] = 0u;
      R.al[i] = 0x3F803F80u;   // alpha = 1 past the end
    }
  }
  R.a8 = (lower_half && tk0 + 8 < n) ? ap[8 * sa] : 0x3F803F80u;
}

// One pass over the chunks of one segment of one (batch, head).
// OUT = true: output pass (state = S, 16 columns per wave, writes o).
// OUT = false: summary pass (state = [S | M], 32 columns per wave).
//
// Per chunk, two factorisations of the pairwise decay e^{g_i - g_j} are used:
//  * fast: one reference at the chunk start, K^ = K e^{g} and K_ = K e^{-g}; valid
//    while every channel decays by less than e^{-80} over the chunk (fp32 and
//    bf16 then hold every factor), chosen per chunk by a block-wide vote;
//  * blocked: references in the middle of each 16-token block, with a per-channel
//    factor e^{m_I - m_J} applied to the column operand of the blocks below the
//    diagonal; valid while log(alpha) >= -11 per token.
template <bool OUT>
__global__ __launch_bounds__(NTHR) void kda_chunk_kernel(ChunkArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Lds& L = *reinterpret_cast<Lds*>(lds_raw);
  constexpr int NCT = OUT ? 1 : 2;        // 16-column state tiles per wave
  constexpr float kFastMin = 1.8e-35f;    // ~e^{-80}

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform
  const int l16 = lane & 15, q4 = lane >> 4;
  const int64_t bh = blockIdx.x / a.P;
  const int p = blockIdx.x % a.P;
  const int64_t b = bh / a.H, h = bh % a.H;
  const int64_t NC = (a.T + CT - 1) / CT;
  const int64_t c_begin = (int64_t)p * a.L;
  const int64_t c_end = min<int64_t>(NC, c_begin + a.L);

  // ---- state init -------------------------------------------------------------
  // wave-owned state tiles S[rt][ct]: rows 16rt + 4q4 + r, column col0 + 16ct + l16
  f32x4 S[8][NCT];
  const int col0 = OUT ? 16 * wave : 32 * (wave & 3);   // column inside S (OUT) or inside S / M (summary)
  const bool m_part = !OUT && wave >= 4;
  {
    const float* src = nullptr;
    if (OUT) src = a.P > 1 ? a.Sstart + ((bh * a.P + p) * D) * D : (a.S0 ? a.S0 + bh * D * D : nullptr);
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * rt + 4 * q4 + r, col = col0 + 16 * ct + l16;
          float s = 0.f;
          if (OUT) {
            if (src) s = src[row * D + col];
          } else if (m_part) {
            s = row == col ? 1.f : 0.f;
          }
          S[rt][ct][r] = s;
        }
  }
  // the blocks of aqk above the diagonal that the output products read stay zero
  for (int e = tid; e < 2 * SBT * SBT; e += NTHR) {
    const int blk = e / (SBT * SBT), i = (e / SBT) % SBT, j = e % SBT;
    const int I = blk == 0 ? 0 : 2, J = I + 1;
    L.aqk[tr(SBT * I + i, SBT * J + j)] = 0;
  }

  // elementwise mapping: wave -> decay block eI and half ehf; lane -> channels ch, ch+1
  const int eI = wave >> 1, ehf = wave & 1;
  const int ch = 2 * lane;
  const int tk0 = SBT * eI + 8 * ehf;

  ChunkRegs R;

  for (int64_t c = c_begin; c < c_end; ++c) {
    const int64_t t0 = c * CT;
    const int n = (int)min<int64_t>(CT, a.T - t0);
    load_chunk<OUT>(a, b, h, t0, n, tk0, ehf == 0, ch, R);
    __syncthreads();   // previous chunk finished with every LDS array

    // ---- E1: norms, decay products relative to block token 8, v^T -----------------
    if (tid < CT) L.beta[tid] = tid < n ? bf2f(a.beta[(b * a.T + t0 + tid) * a.H + h]) : 0.f;
    if (a.l2norm) {
      float ss[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float k0 = bf_lo(R.k[i]), k1 = bf_hi(R.k[i]);
        const float q0 = bf_lo(R.q[i]), q1 = bf_hi(R.q[i]);
        ss[i] = k0 * k0 + k1 * k1;
        ss[i + 8] = q0 * q0 + q1 * q1;
      }
      const float tot = wave_sum16(ss, lane);
      if ((lane & 3) == 0) {
        const int vv = lane >> 2;                 // 0..7: k of token vv; 8..15: q of token vv - 8
        const float rn = __builtin_amdgcn_rsqf(tot + kL2Eps);
        if (vv < 8) L.rk[tk0 + vv] = rn; else L.rq[tk0 + vv - 8] = rn;
      }
    } else if (lane < 8) {
      L.rk[tk0 + lane] = 1.f;
      L.rq[tk0 + lane] = 1.f;
    }
    // er = e^{g - m_I}, ec = 1 / er, m_I = g at the block's token 8
    float er[8][2], ec[8][2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      if (ehf == 1) {
        float run = 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          if (i > 0) run *= cc ? bf_hi(R.al[i]) : bf_lo(R.al[i]);
          er[i][cc] = run;
          ec[i][cc] = __builtin_amdgcn_rcpf(run);
        }
        L.pf[eI][ch + cc] = run;
      } else {
        float run = cc ? bf_hi(R.a8) : bf_lo(R.a8);
#pragma unroll
        for (int i = 7; i >= 0; --i) {
          if (i < 7) run *= cc ? bf_hi(R.al[i + 1]) : bf_lo(R.al[i + 1]);
          ec[i][cc] = run;
          er[i][cc] = __builtin_amdgcn_rcpf(run);
        }
        L.pb[eI][ch + cc] = run * (cc ? bf_hi(R.al[0]) : bf_lo(R.al[0]));
      }
    }
    {  // v^T: channel ch and ch+1, 8 consecutive tokens each
      uint4 lo, hi;
      lo.x = (R.v[0] & 0xffffu) | (R.v[1] << 16); hi.x = (R.v[0] >> 16) | (R.v[1] & 0xffff0000u);
      lo.y = (R.v[2] & 0xffffu) | (R.v[3] << 16); hi.y = (R.v[2] >> 16) | (R.v[3] & 0xffff0000u);
      lo.z = (R.v[4] & 0xffffu) | (R.v[5] << 16); hi.z = (R.v[4] >> 16) | (R.v[5] & 0xffff0000u);
      lo.w = (R.v[6] & 0xffffu) | (R.v[7] << 16); hi.w = (R.v[6] >> 16) | (R.v[7] & 0xffff0000u);
      *reinterpret_cast<uint4*>(&L.vT[tr(ch, tk0)]) = lo;
      *reinterpret_cast<uint4*>(&L.vT[tr(ch + 1, tk0)]) = hi;
    }
    __syncthreads();

    // ---- E2: block decay factors of this wave's block and channels, in registers -------
    // full_J = product of alpha over block J; em = e^{m_I}, iem = e^{-m_I},
    // enm = e^{g_n - m_I}, egn = e^{g_n}. Every wave holds all 128 channels, so every
    // wave reaches the same vote for the fast factorisation.
    float em2[2], iem2[2], enm2[2], egn2[2];
    {
      float pbv[NSB][2], pfv[NSB][2], full[NSB][2];
#pragma unroll
      for (int J = 0; J < NSB; ++J) {
        const float2 pb2 = *reinterpret_cast<const float2*>(&L.pb[J][ch]);
        const float2 pf2 = *reinterpret_cast<const float2*>(&L.pf[J][ch]);
        pbv[J][0] = pb2.x; pbv[J][1] = pb2.y; pfv[J][0] = pf2.x; pfv[J][1] = pf2.y;
        full[J][0] = pb2.x * pf2.x; full[J][1] = pb2.y * pf2.y;
      }
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        float pre = 1.f, post = 1.f, all = 1.f;
#pragma unroll
        for (int J = 0; J < NSB; ++J) {
          if (J < eI) pre *= full[J][cc];
          if (J > eI) post *= full[J][cc];
          all *= full[J][cc];
        }
        float pbI = pbv[0][cc], pfI = pfv[0][cc];
#pragma unroll
        for (int J = 1; J < NSB; ++J) if (J == eI) { pbI = pbv[J][cc]; pfI = pfv[J][cc]; }
        em2[cc] = pre * pbI;
        iem2[cc] = __builtin_amdgcn_rcpf(em2[cc]);
        enm2[cc] = pfI * post;
        egn2[cc] = all;
      }
      if (wave == 0) {
        *reinterpret_cast<float2*>(&L.egn[ch]) = make_float2(egn2[0], egn2[1]);
#pragma unroll
        for (int I = 1; I < NSB; ++I) {
          float mid0 = 1.f, mid1 = 1.f;
#pragma unroll
          for (int J = I - 1; J >= 0; --J) {
            *reinterpret_cast<float2*>(&L.pij[pair_index(I, J)][ch]) =
                make_float2(pfv[J][0] * mid0 * pbv[I][0], pfv[J][1] * mid1 * pbv[I][1]);
            mid0 *= full[J][0];
            mid1 *= full[J][1];
          }
        }
      }
    }
    const bool fast = __all(egn2[0] >= kFastMin && egn2[1] >= kFastMin) != 0;

    // ---- E3: MFMA operands ------------------------------------------------------------
    {
      float kf[8][2], qf[8][2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        kf[i][0] = bf_lo(R.k[i]); kf[i][1] = bf_hi(R.k[i]);
        qf[i][0] = bf_lo(R.q[i]); qf[i][1] = bf_hi(R.q[i]);
      }
      const float em0 = em2[0], em1 = em2[1];
      uint32_t kb0[4], kb1[4], kt0[4], kt1[4];
      if (fast) {
        // K^ = K e^{g} (row operand of A and right-hand side of W), K_ = K e^{-g},
        // K~ = K_ e^{g_n}, Q^ = Q e^{g} (row operand of Aqk and of Q^ S)
        const float iem0 = iem2[0], iem1 = iem2[1];
        const float gn0 = egn2[0], gn1 = egn2[1];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          float kh[2][2], kl[2][2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const float f0 = er[i + u][0] * em0, f1 = er[i + u][1] * em1;
            const float g0 = ec[i + u][0] * iem0, g1 = ec[i + u][1] * iem1;
            kh[u][0] = kf[i + u][0] * f0; kh[u][1] = kf[i + u][1] * f1;
            kl[u][0] = kf[i + u][0] * g0; kl[u][1] = kf[i + u][1] * g1;
            *reinterpret_cast<uint32_t*>(&L.kr[rm(tk0 + i + u, ch)]) = pack_bf16x2(kh[u][0], kh[u][1]);
            *reinterpret_cast<uint32_t*>(&L.kc[rm(tk0 + i + u, ch)]) = pack_bf16x2(kl[u][0], kl[u][1]);
            if (OUT)
              *reinterpret_cast<uint32_t*>(&L.qh[rm(tk0 + i + u, ch)]) =
                  pack_bf16x2(qf[i + u][0] * f0, qf[i + u][1] * f1);
          }
          kb0[i / 2] = pack_bf16x2(kh[0][0], kh[1][0]);
          kb1[i / 2] = pack_bf16x2(kh[0][1], kh[1][1]);
          kt0[i / 2] = pack_bf16x2(kl[0][0] * gn0, kl[1][0] * gn0);
          kt1[i / 2] = pack_bf16x2(kl[0][1] * gn1, kl[1][1] * gn1);
        }
      } else {
        const float enm0 = enm2[0], enm1 = enm2[1];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          float kh[2][2], kl[2][2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
              kh[u][cc] = kf[i + u][cc] * er[i + u][cc];
              kl[u][cc] = kf[i + u][cc] * ec[i + u][cc];
            }
            const float qr0 = qf[i + u][0] * er[i + u][0], qr1 = qf[i + u][1] * er[i + u][1];
            *reinterpret_cast<uint32_t*>(&L.kr[rm(tk0 + i + u, ch)]) = pack_bf16x2(kh[u][0], kh[u][1]);
            *reinterpret_cast<uint32_t*>(&L.kc[rm(tk0 + i + u, ch)]) = pack_bf16x2(kl[u][0], kl[u][1]);
            if (OUT) {
              *reinterpret_cast<uint32_t*>(&L.qr[rm(tk0 + i + u, ch)]) = pack_bf16x2(qr0, qr1);
              *reinterpret_cast<uint32_t*>(&L.qh[rm(tk0 + i + u, ch)]) = pack_bf16x2(qr0 * em0, qr1 * em1);
            }
          }
          kb0[i / 2] = pack_bf16x2(kh[0][0] * em0, kh[1][0] * em0);
          kb1[i / 2] = pack_bf16x2(kh[0][1] * em1, kh[1][1] * em1);
          kt0[i / 2] = pack_bf16x2(kl[0][0] * enm0, kl[1][0] * enm0);
          kt1[i / 2] = pack_bf16x2(kl[0][1] * enm1, kl[1][1] * enm1);
        }
      }
      *reinterpret_cast<uint4*>(&L.kbT[tr(ch, tk0)]) = make_uint4(kb0[0], kb0[1], kb0[2], kb0[3]);
      *reinterpret_cast<uint4*>(&L.kbT[tr(ch + 1, tk0)]) = make_uint4(kb1[0], kb1[1], kb1[2], kb1[3]);
      *reinterpret_cast<uint4*>(&L.ktT[tr(ch, tk0)]) = make_uint4(kt0[0], kt0[1], kt0[2], kt0[3]);
      *reinterpret_cast<uint4*>(&L.ktT[tr(ch + 1, tk0)]) = make_uint4(kt1[0], kt1[1], kt1[2], kt1[3]);
    }
    __syncthreads();

    // ---- M1 + T: A and Aqk blocks; diagonal inverses; Q^ S for the output ------------
    // Waves 0-3 compute A(I, I) for I = wave and invert that block right away (the
    // same wave wrote it, so no block barrier is needed); waves 4-7 compute the Aqk
    // diagonal blocks and every block below the diagonal.
    f32x4 O[4];
    auto qs_product = [&]() {
      uint4 Sf0[4], qf[4][4];
#pragma unroll
      for (int s = 0; s < 4; ++s) Sf0[s] = pack8(S[2 * s][0], S[2 * s + 1][0]);
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[I][s] = ld_perm(L.qh, rm(SBT * I + l16, 0), 32 * s + 4 * q4);
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mma32(qf[I][s], Sf0[s], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= L.rq[SBT * I + 4 * q4 + r];
        O[I] = acc;
      }
    };
    {
      auto tile = [&](bool is_a, int I, int J) {
        const uint16_t* rowop = is_a ? L.kr : (fast ? L.qh : L.qr);
        uint4 af[4], bfr[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          af[s] = ld128(rowop, rm(SBT * I + l16, 32 * s + 8 * q4));
          bfr[s] = ld128(L.kc, rm(SBT * J + l16, 32 * s + 8 * q4));
        }
        if (!fast && I != J) {
          const float* pp = &L.pij[pair_index(I, J)][8 * q4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float4 p0 = *reinterpret_cast<const float4*>(pp + 32 * s);
            const float4 p1 = *reinterpret_cast<const float4*>(pp + 32 * s + 4);
            const uint4 u = bfr[s];
            bfr[s] = make_uint4(pack_bf16x2(bf_lo(u.x) * p0.x, bf_hi(u.x) * p0.y),
                                pack_bf16x2(bf_lo(u.y) * p0.z, bf_hi(u.y) * p0.w),
                                pack_bf16x2(bf_lo(u.z) * p1.x, bf_hi(u.z) * p1.y),
                                pack_bf16x2(bf_lo(u.w) * p1.z, bf_hi(u.w) * p1.w));
          }
        }
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mma32(af[s], bfr[s], acc);
        const int j = SBT * J + l16;
        const float rkj = L.rk[j];
        float val[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = SBT * I + 4 * q4 + r;
          const float rowf = is_a ? L.beta[i] * L.rk[i] : L.rq[i];
          const bool keep = is_a ? i > j : i >= j;
          val[r] = keep ? rowf * rkj * acc[r] : 0.f;
        }
        if (is_a && I == J) {
#pragma unroll
          for (int r = 0; r < 4; ++r) L.adiag[I][4 * q4 + r][4 * (l16 & 3) + (l16 >> 2)] = val[r];   // k-interleaved
        } else {
          uint16_t* dst = is_a ? L.at : L.aqk;
          const float sg = is_a ? -1.f : 1.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[tr(SBT * I + 4 * q4 + r, j)] = f2bf(sg * val[r]);
        }
      };
      if (wave < 4) {
        const int I = wave;
        tile(true, I, I);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // forward substitution: lane = 16 part + j owns column j and the terms
        // k = part + 4m of every row's sum; the four parts are summed with lane swaps
        const int part = lane >> 4, jj = lane & 15;
        float xs[4] = {0.f, 0.f, 0.f, 0.f};   // x[part + 4m] of column jj
        float4 arow[SBT];
#pragma unroll
        for (int i = 0; i < SBT; ++i) arow[i] = *reinterpret_cast<const float4*>(&L.adiag[I][i][4 * part]);
#pragma unroll
        for (int i = 0; i < SBT; ++i) {
          float ps = arow[i].x * xs[0] + arow[i].y * xs[1] + arow[i].z * xs[2] + arow[i].w * xs[3];
          ps = halve16(ps, ps);
          ps = halve32(ps, ps);
          const float xi = (i == jj ? 1.f : 0.f) - ps;
          if (part == (i & 3)) xs[i >> 2] = xi;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) L.at[tr(SBT * I + part + 4 * m, SBT * I + jj)] = f2bf(xs[m]);
      } else {
        const int w4 = wave - 4;
        if (OUT) tile(false, w4, w4);
        // pairs (I, J), I > J: waves 4, 5 take two, waves 6, 7 one
        constexpr int PI[6] = {1, 2, 2, 3, 3, 3};
        constexpr int PJ[6] = {0, 0, 1, 0, 1, 2};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int pi = u == 0 ? w4 : w4 + 4;
          if (pi < 6) {
            tile(true, PI[pi], PJ[pi]);
            if (OUT) tile(false, PI[pi], PJ[pi]);
          }
        }
      }
      if (OUT) qs_product();
    }
    __syncthreads();

    uint4 Sf[4][NCT];   // state as bf16 B operand, K permuted: slots 0-3 rows 32s+4q+r, 4-7 rows 32s+16+4q+r
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) Sf[s][ct] = pack8(S[2 * s][ct], S[2 * s + 1][ct]);

    // ---- X: block substitution X = (I + A)^{-1} diag(sigma) R -------------------------
    // right-hand sides: OUT -> wave w: V tile w (U~, kept) and Kb tile w (W, to LDS)
    //                   summary -> waves 0-3: V tiles 2w, 2w+1; waves 4-7: Kb tiles 2(w-4), 2(w-4)+1
    f32x4 U[4][NCT];   // U~ from the substitution, then U = U~ - W S in place
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) U[I][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      constexpr int NJOB = 2;
#pragma unroll
      for (int job = 0; job < NJOB; ++job) {
        bool is_v;
        int ctile;
        if (OUT) { is_v = job == 0; ctile = wave; }
        else { is_v = wave < 4; ctile = 2 * (wave & 3) + job; }
        const uint16_t* RT = is_v ? L.vT : L.kbT;
        f32x4 X[4];
        uint2 Xb[4];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
          const uint2 raw = *reinterpret_cast<const uint2*>(&RT[tr(SBT * ctile + l16, SBT * I + 4 * q4)]);
          f32x4 y;
          y[0] = bf_lo(raw.x); y[1] = bf_hi(raw.x); y[2] = bf_lo(raw.y); y[3] = bf_hi(raw.y);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = SBT * I + 4 * q4 + r;
            y[r] *= is_v ? L.beta[i] : L.beta[i] * L.rk[i];
          }
#pragma unroll
          for (int J = 0; J < I; ++J) {
            const uint2 af = *reinterpret_cast<const uint2*>(&L.at[tr(SBT * I + l16, SBT * J + 4 * q4)]);
            y = mma16(af, Xb[J], y);
          }
          const uint2 tf = *reinterpret_cast<const uint2*>(&L.at[tr(SBT * I + l16, SBT * I + 4 * q4)]);
          X[I] = mma16(tf, pack4(y), f32x4{0.f, 0.f, 0.f, 0.f});
          Xb[I] = pack4(X[I]);
        }
        if (is_v) {
          const int ct = OUT ? 0 : job;
#pragma unroll
          for (int I = 0; I < 4; ++I) U[I][ct] = X[I];
        } else {
#pragma unroll
          for (int I = 0; I < 4; ++I)
#pragma unroll
            for (int r = 0; r < 4; ++r) L.kr[rm(SBT * I + 4 * q4 + r, SBT * ctile + l16)] = f2bf(-X[I][r]);
        }
      }
    }
    __syncthreads();

    // ---- S: U = U~ - W S;  O += Aqk U;  S <- Diag(e^{g_n}) S + K~^T diag(1/|k|) U --------
    if (OUT) {   // all W fragments in flight together
      uint4 wf[4][4];
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int s = 0; s < 4; ++s) wf[I][s] = ld_perm(L.kr, rm(SBT * I + l16, 0), 32 * s + 4 * q4);
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int s = 0; s < 4; ++s) U[I][0] = mma32(wf[I][s], Sf[s][0], U[I][0]);
    } else {     // the summary pass holds twice the state: one row block of W at a time
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        uint4 wf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) wf[s] = ld_perm(L.kr, rm(SBT * I + l16, 0), 32 * s + 4 * q4);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int s = 0; s < 4; ++s) U[I][ct] = mma32(wf[s], Sf[s][ct], U[I][ct]);
      }
    }
    if (OUT) {
      uint4 Uf[2], af[6];
#pragma unroll
      for (int s = 0; s < 2; ++s) Uf[s] = pack8(U[2 * s][0], U[2 * s + 1][0]);
      af[0] = ld_perm(L.aqk, tr(l16, 0), 4 * q4);
      af[1] = ld_perm(L.aqk, tr(SBT + l16, 0), 4 * q4);
      af[2] = ld_perm(L.aqk, tr(2 * SBT + l16, 0), 4 * q4);
      af[3] = ld_perm(L.aqk, tr(2 * SBT + l16, 0), 32 + 4 * q4);
      af[4] = ld_perm(L.aqk, tr(3 * SBT + l16, 0), 4 * q4);
      af[5] = ld_perm(L.aqk, tr(3 * SBT + l16, 0), 32 + 4 * q4);
      O[0] = mma32(af[0], Uf[0], O[0]);
      O[1] = mma32(af[1], Uf[0], O[1]);
      O[2] = mma32(af[2], Uf[0], O[2]);
      O[2] = mma32(af[3], Uf[1], O[2]);
      O[3] = mma32(af[4], Uf[0], O[3]);
      O[3] = mma32(af[5], Uf[1], O[3]);
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) L.qr[rm(SBT * I + 4 * q4 + r, 16 * wave + l16)] = f2bf(O[I][r]);
    }
    {
      // scale U rows by 1/|k| for the state update
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float rk = L.rk[SBT * I + 4 * q4 + r];
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) U[I][ct][r] *= rk;
        }
      uint4 Upf[2][NCT];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Upf[s][ct] = pack8(U[2 * s][ct], U[2 * s + 1][ct]);
      constexpr int NKB = OUT ? 8 : 2;   // row tiles of K~^T fragments loaded ahead
      uint4 kf2[8][2];
#pragma unroll
      for (int rt = 0; rt < NKB; ++rt)
#pragma unroll
        for (int s = 0; s < 2; ++s) kf2[rt][s] = ld_perm(L.ktT, tr(SBT * rt + l16, 0), 32 * s + 4 * q4);
#pragma unroll
      for (int rt = 0; rt < 8; ++rt) {
        if (rt + NKB < 8) {
#pragma unroll
          for (int s = 0; s < 2; ++s) kf2[rt + NKB][s] = ld_perm(L.ktT, tr(SBT * (rt + NKB) + l16, 0), 32 * s + 4 * q4);
        }
        float dec[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) dec[r] = L.egn[SBT * rt + 4 * q4 + r];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          f32x4 acc = S[rt][ct];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] *= dec[r];
#pragma unroll
          for (int s = 0; s < 2; ++s) acc = mma32(kf2[rt][s], Upf[s][ct], acc);
          S[rt][ct] = acc;
        }
      }
    }
    if (OUT) {
      __syncthreads();
      // output tile rows -> o[b, t0 + row, h, :]
      const int row = tid >> 3, seg = tid & 7;
      if (row < n) {
        uint16_t* dst = a.o + ((b * a.T + t0 + row) * a.H + h) * D + 16 * seg;
        reinterpret_cast<uint4*>(dst)[0] = *reinterpret_cast<const uint4*>(&L.qr[rm(row, 16 * seg)]);
        reinterpret_cast<uint4*>(dst)[1] = *reinterpret_cast<const uint4*>(&L.qr[rm(row, 16 * seg + 8)]);
      }
    }
  }

  // ---- write back ------------------------------------------------------------------
  if (OUT) {
    if (a.S_final != nullptr && p == a.P - 1) {
#pragma unroll
      for (int rt = 0; rt < 8; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          a.S_final[(bh * D + 16 * rt + 4 * q4 + r) * D + col0 + l16] = S[rt][0][r];
    }
  } else {
    float* dst = a.SM + ((bh * a.P + p) * D) * (2 * D);
    const int acol = (m_part ? D : 0) + col0;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * rt + 4 * q4 + r) * (2 * D) + acol + 16 * ct + l16] = S[rt][ct][r];
  }
}

// S_start(0) = S0 (or 0); S_start(p+1) = M_p S_start(p) + S_p, for p < P - 1.
// One block per (batch, head), 8 waves; wave w owns state columns 16w..16w+15
// in registers (fp32). M_p is staged in LDS split into bf16 high and low parts
// and the product is formed from three bf16 MFMAs (hi*hi + hi*lo + lo*hi) with
// fp32 accumulation, about 16 significant bits per product; the next M_p is
// prefetched into registers while the current one is used.
constexpr int MS = D + 8;    // padded row of the staged M (bf16 elements)

__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}

__global__ __launch_bounds__(NTHR) void kda_combine_kernel(const float* __restrict__ SM, const float* __restrict__ S0,
                                                           float* __restrict__ Sstart, int P) {
  __shared__ __align__(16) uint16_t mhi[D * MS];
  __shared__ __align__(16) uint16_t mlo[D * MS];
  const int64_t bh = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = 16 * wave + l16;

  f32x4 S[8];
#pragma unroll
  for (int rt = 0; rt < 8; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[rt][r] = S0 ? S0[(bh * D + 16 * rt + 4 * q4 + r) * D + col] : 0.f;

  // thread t stages rows (t >> 5) + 16 j of M, columns 4 (t & 31) .. +3
  const int mrow = tid >> 5, mcol = 4 * (tid & 31);
  float4 pre[8];
  auto fetch = [&](int p) {
    const float* m = SM + ((bh * P + p) * D) * (2 * D) + D;
#pragma unroll
    for (int j = 0; j < 8; ++j) pre[j] = *reinterpret_cast<const float4*>(m + (mrow + 16 * j) * (2 * D) + mcol);
  };
  if (P > 1) fetch(0);
  for (int p = 0; p < P; ++p) {
    float* outp = Sstart + ((bh * P + p) * D) * D;
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) outp[(16 * rt + 4 * q4 + r) * D + col] = S[rt][r];
    if (p == P - 1) break;
    __syncthreads();   // previous M fully consumed
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = mrow + 16 * j;
      uint16_t h0, l0, h1, l1, h2, l2, h3, l3;
      split_bf16(pre[j].x, h0, l0); split_bf16(pre[j].y, h1, l1);
      split_bf16(pre[j].z, h2, l2); split_bf16(pre[j].w, h3, l3);
      *reinterpret_cast<uint2*>(&mhi[row * MS + mcol]) =
          make_uint2(uint32_t(h0) | (uint32_t(h1) << 16), uint32_t(h2) | (uint32_t(h3) << 16));
      *reinterpret_cast<uint2*>(&mlo[row * MS + mcol]) =
          make_uint2(uint32_t(l0) | (uint32_t(l1) << 16), uint32_t(l2) | (uint32_t(l3) << 16));
    }
    __syncthreads();
    if (p + 2 < P) fetch(p + 1);
    // B operand: the state split into hi and lo, K permuted as in the chunk kernel
    uint4 bh_[4], bl_[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f32x4 lo0, lo1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lo0[r] = S[2 * s][r] - bf2f(f2bf(S[2 * s][r]));
        lo1[r] = S[2 * s + 1][r] - bf2f(f2bf(S[2 * s + 1][r]));
      }
      bh_[s] = pack8(S[2 * s], S[2 * s + 1]);
      bl_[s] = pack8(lo0, lo1);
    }
    const float* sp = SM + ((bh * P + p) * D) * (2 * D);
    f32x4 acc[8];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rt][r] = sp[(16 * rt + 4 * q4 + r) * (2 * D) + col];
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int row = 16 * rt + l16;
        const uint4 ah = cat(*reinterpret_cast<const uint2*>(&mhi[row * MS + 32 * s + 4 * q4]),
                             *reinterpret_cast<const uint2*>(&mhi[row * MS + 32 * s + 16 + 4 * q4]));
        const uint4 al = cat(*reinterpret_cast<const uint2*>(&mlo[row * MS + 32 * s + 4 * q4]),
                             *reinterpret_cast<const uint2*>(&mlo[row * MS + 32 * s + 16 + 4 * q4]));
        acc[rt] = mma32(al, bh_[s], acc[rt]);
        acc[rt] = mma32(ah, bl_[s], acc[rt]);
        acc[rt] = mma32(ah, bh_[s], acc[rt]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < 8; ++rt) S[rt] = acc[rt];
  }
}

struct Split {
  int P, L;
};

Split choose_split(int64_t B, int64_t T, int64_t H, bool no_split) {
  const int64_t NC = (T + CT - 1) / CT;
  const int64_t BH = B * H;
  if (no_split || NC <= 1 || BH >= kTargetBlocks) return Split{1, (int)NC};
  int64_t P = (kTargetBlocks + BH - 1) / BH;
  if (P > NC) P = NC;
  const int64_t Lc = (NC + P - 1) / P;
  P = (NC + Lc - 1) / Lc;
  return Split{(int)P, (int)Lc};
}

}  // namespace

bool kda_chunked_supported(const KdaArgs& a) { return a.bf16 && a.dk == D && a.dv == D; }

int64_t kda_chunked_segments(int64_t B, int64_t T, int64_t H, bool no_split) {
  return choose_split(B, T, H, no_split).P;
}

size_t kda_chunked_workspace(int64_t B, int64_t T, int64_t H, bool no_split) {
  const Split sp = choose_split(B, T, H, no_split);
  if (sp.P <= 1) return 0;
  const size_t per = (size_t)D * (2 * D) * sizeof(float) + (size_t)D * D * sizeof(float);
  return (size_t)(B * H) * sp.P * per;
}

hipError_t launch_kda_chunked(const KdaArgs& x, bool no_split, void* workspace, hipStream_t stream) {
  const Split sp = choose_split(x.B, x.T, x.H, no_split);
  const int64_t BH = x.B * x.H;
  if (BH * sp.P > 0x7fffffff) return hipErrorInvalidValue;
  ChunkArgs a;
  a.q = static_cast<const uint16_t*>(x.q);
  a.k = static_cast<const uint16_t*>(x.k);
  a.v = static_cast<const uint16_t*>(x.v);
  a.stride = x.qkv_stride;
  a.alpha = static_cast<const uint16_t*>(x.alpha);
  a.beta = static_cast<const uint16_t*>(x.beta);
  a.S0 = x.S0;
  a.Sstart = nullptr;
  a.SM = nullptr;
  a.o = static_cast<uint16_t*>(x.o);
  a.S_final = x.S_final;
  a.T = x.T;
  a.H = x.H;
  a.P = sp.P;
  a.L = sp.L;
  a.l2norm = x.l2norm ? 1 : 0;
  const size_t lds = sizeof(Lds);
  int dev = 0;
  hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  static bool attr_done[64] = {};
  if (dev < 0 || dev >= 64 || !attr_done[dev]) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < 64) attr_done[dev] = true;
  }
  if (sp.P > 1) {
    float* SM = static_cast<float*>(workspace);
    float* Sst = SM + (size_t)BH * sp.P * D * (2 * D);
    a.SM = SM;
    hipLaunchKernelGGL(kda_chunk_kernel<false>, dim3((unsigned)(BH * sp.P)), dim3(NTHR), lds, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kda_combine_kernel, dim3((unsigned)BH), dim3(NTHR), 0, stream, SM, x.S0, Sst, sp.P);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    a.Sstart = Sst;
  }
  hipLaunchKernelGGL(kda_chunk_kernel<true>, dim3((unsigned)(BH * sp.P)), dim3(NTHR), lds, stream, a);
  return hipGetLastError();
}

}  // namespace chm
