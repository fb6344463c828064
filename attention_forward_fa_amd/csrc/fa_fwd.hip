// Fused attention forward for MI355X (gfx950, CDNA4): kernels and the C ABI
// declared in include/fa_mi355x.h.
//
// Method: query tiles stay on chip while K/V blocks stream past them; a
// running row max and row sum rescale the output accumulator whenever the max
// grows, and the accumulator is divided by the row sum at the end (the online
// softmax of "TCA 51%，MFU 不足 8%", section "FA2 TCA 虚高归因", and the
// consumer loop of "第 17 章 TMA + Warp Specialization 把 FA2 写到 SOTA" §17.5).
// The N x N scores never leave registers.
//
// gfx950 mapping (the pages' TMA / mbarrier / WGMMA / TMEM machinery has no
// counterpart here and is not imitated):
//   * workgroup = 4 waves of 64 lanes; each wave owns 32 query rows, so a
//     workgroup covers BR = 128 rows of one (b, h) head;
//   * K/V blocks of BC = 64 keys are staged global -> VGPR -> LDS; the global
//     loads for block j+1 are in flight while block j is computed;
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16} (or the fp8 v_mfma_scale_f32_32x32x64
//     with unit block scales).  In the 32x32 accumulator layout a lane owns
//     one column (= one query) and 16 rows (= keys), so the row max / row sum
//     of the softmax are in-lane reductions plus one exchange with the lane
//     32 apart (v_permlane32_swap);
//   * the same accumulator registers, rounded to fp16, are already the B
//     operand of O^T += V^T P^T: the key order inside one MFMA's contraction
//     is free, so P never moves between lanes or through LDS;
//   * V is transposed (and converted to fp16) while it is staged, so the A
//     operand of the PV product is two 8-byte LDS reads per lane;
//   * LDS rows are padded so the operand reads are free of bank conflicts.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa_mi355x.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kQW = 32;            // query rows per wave
constexpr int kBR = kQW * kWaves;  // query rows per workgroup
constexpr int kBC = 64;            // keys per K/V block
constexpr int kKPad = 16;          // bytes of padding per K row in LDS
constexpr int kVPad = 4;           // halfs of padding per V^T row in LDS
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Input element type: 0 fp16, 1 bf16, 2 fp8 e4m3.
template <int DT>
struct Elem {
  static constexpr int bytes = (DT == FA_DTYPE_FP8_E4M3) ? 1 : 2;
  // Contraction depth of one QK^T MFMA and the per-lane operand size.
  static constexpr int kstep = (DT == FA_DTYPE_FP8_E4M3) ? 64 : 16;
  static constexpr int opnd_dwords = (DT == FA_DTYPE_FP8_E4M3) ? 8 : 4;
};

template <int DT>
struct QKOperand {
  uint32_t w[Elem<DT>::opnd_dwords];
};

template <int DT>
__device__ __forceinline__ f32x16 mfma_qk(const QKOperand<DT>& a, const QKOperand<DT>& b,
                                          f32x16 c) {
  if constexpr (DT == FA_DTYPE_FP16) {
    u32x4 ua = {a.w[0], a.w[1], a.w[2], a.w[3]};
    u32x4 ub = {b.w[0], b.w[1], b.w[2], b.w[3]};
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ua),
                                                  __builtin_bit_cast(f16x8, ub), c, 0, 0, 0);
  } else if constexpr (DT == FA_DTYPE_BF16) {
    u32x4 ua = {a.w[0], a.w[1], a.w[2], a.w[3]};
    u32x4 ub = {b.w[0], b.w[1], b.w[2], b.w[3]};
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ua),
                                                   __builtin_bit_cast(bf16x8, ub), c, 0, 0, 0);
  } else {
    i32x8 ia, ib;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ia[i] = (int)a.w[i];
      ib[i] = (int)b.w[i];
    }
    // Operand formats 0/0 = OCP E4M3 for A and B; E8M0 block scale 127 = 2^0.
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ia, ib, c, 0, 0, 0, 127, 0, 127);
  }
}

__device__ __forceinline__ f32x16 mfma_pv(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Lanes l and l^32 hold the same query.  v_permlane32_swap with both operands
// equal to x leaves each lane holding {x[l], x[l^32]} across its two results,
// so a symmetric combination of the pair reduces over the two lanes.
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 h = {(_Float16)lo, (_Float16)hi};  // v_cvt_pk_f16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

// Two consecutive storage elements of V (one dword, fp16 or bf16) as fp16x2;
// or, for fp8, two e4m3 codes from the low / high 16 bits of a dword.
template <int DT, bool HI_WORD>
__device__ __forceinline__ uint32_t v_pair_to_f16(uint32_t w) {
  if constexpr (DT == FA_DTYPE_FP16) {
    return w;
  } else if constexpr (DT == FA_DTYPE_BF16) {
    // bf16 -> fp32 is exact (upper half of a binary32); fp32 -> fp16 is exact for
    // every |v| in [2^-14, 65504] and rounds to nearest even below that.
    float lo = __uint_as_float(w << 16);
    float hi = __uint_as_float(w & 0xffff0000u);
    return pack_f16x2(lo, hi);
  } else {
    f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI_WORD);  // exact
    return __builtin_bit_cast(uint32_t, h);
  }
}

struct Params {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* descale_q;  // NULL: unit scales
  const float* descale_k;
  const float* descale_v;
  _Float16* o;
  float* lse;
  int H;
  int N;
  int n_qtiles;
  int bh;  // B*H
  float scale;
};

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void fa_fwd_kernel(Params p) {
  using E = Elem<DT>;
  constexpr int ES = E::bytes;
  constexpr int KROW = D * ES + kKPad;          // bytes per K row in LDS
  constexpr int VROW = kBC + kVPad;             // halfs per V^T row in LDS
  constexpr int NKS = D / E::kstep;             // QK^T MFMAs per 32x32 tile
  constexpr int NDT = D / 32;                   // 32-wide d tiles of O^T
  constexpr int K_CHUNKS = kBC * D * ES / 16;   // 16-byte chunks in a K block
  constexpr int K_PER_T = K_CHUNKS / kThreads;  // per thread
  constexpr int K_CHUNKS_ROW = D * ES / 16;
  constexpr int VD = D / 16;                    // d values per thread in V staging
  constexpr int VBYTES = VD * ES;               // bytes per key row per thread
  constexpr int VWORDS = (VBYTES + 3) / 4;
  static_assert(K_CHUNKS % kThreads == 0, "K staging must tile the workgroup");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kBC * KROW];
  __shared__ __attribute__((aligned(16))) _Float16 vt_lds[D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 31;   // row/column index inside a 32x32 MFMA tile
  const int hh = lane >> 5;   // which half of the wave

  // ---- work decomposition: one workgroup per (b*H + h, query tile) ----------
  const int wg = blockIdx.x;
  int bh, qt;
  if constexpr (CAUSAL) {
    // Longest tiles first: the last query tile of every head, then the one
    // before it, and so on.
    bh = wg % p.bh;
    qt = p.n_qtiles - 1 - wg / p.bh;
  } else {
    bh = wg / p.n_qtiles;
    qt = wg % p.n_qtiles;
  }
  const int N = p.N;
  const int64_t head_off = (int64_t)bh * N * D;
  const uint8_t* qg = p.q + head_off * ES;
  const uint8_t* kg = p.k + head_off * ES;
  const uint8_t* vg = p.v + head_off * ES;

  const int q0 = qt * kBR;                 // first query row of the workgroup
  const int qw0 = q0 + wave * kQW;         // first query row of this wave
  const int my_q = qw0 + lr;               // the query this lane's column holds

  float c = p.scale * kLog2e;  // exp(x) = exp2(x * log2 e)
  float v_scale = 1.0f;
  if constexpr (DT == FA_DTYPE_FP8_E4M3) {
    if (p.descale_q) {
      c *= p.descale_q[bh] * p.descale_k[bh];
      v_scale = p.descale_v[bh];
    }
  }

  // ---- Q tile -> registers, laid out as the B operand of S^T = K Q^T ---------
  QKOperand<DT> qreg[NKS];
  {
    const bool ok = my_q < N;
    const uint8_t* src = qg + (int64_t)(ok ? my_q : 0) * D * ES;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int byte = (ks * E::kstep + hh * (E::kstep / 2)) * ES;
#pragma unroll
      for (int w = 0; w < E::opnd_dwords; w += 4) {
        u32x4 x = ok ? *reinterpret_cast<const u32x4*>(src + byte + 4 * w) : u32x4{0, 0, 0, 0};
        qreg[ks].w[w + 0] = x[0];
        qreg[ks].w[w + 1] = x[1];
        qreg[ks].w[w + 2] = x[2];
        qreg[ks].w[w + 3] = x[3];
      }
    }
  }

  // ---- number of K/V blocks this workgroup visits -----------------------------
  int kv_end = N;
  if constexpr (CAUSAL) kv_end = min(N, q0 + kBR);
  const int nblk = (kv_end + kBC - 1) / kBC;

  // ---- staging registers ----------------------------------------------------
  u32x4 kst[K_PER_T];
  uint32_t vst[4][VWORDS];
  const int va = tid / 16;  // keys 4*va .. 4*va+3 of the block
  const int vc = tid % 16;  // d values vc*VD .. vc*VD+VD-1

  auto load_block = [&](int kb) {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / K_CHUNKS_ROW;
      const int col = ch % K_CHUNKS_ROW;
      const int key = kb + row;
      kst[i] = key < N ? *reinterpret_cast<const u32x4*>(kg + ((int64_t)key * D * ES) + col * 16)
                       : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kb + 4 * va + r;
      const uint8_t* src = vg + (int64_t)key * D * ES + vc * VBYTES;
      if constexpr (VBYTES == 16) {
        u32x4 x = key < N ? *reinterpret_cast<const u32x4*>(src) : u32x4{0, 0, 0, 0};
        vst[r][0] = x[0]; vst[r][1] = x[1]; vst[r][2] = x[2]; vst[r][3] = x[3];
      } else if constexpr (VBYTES == 8) {
        u32x2 x = key < N ? *reinterpret_cast<const u32x2*>(src) : u32x2{0, 0};
        vst[r][0] = x[0]; vst[r][1] = x[1];
      } else {
        vst[r][0] = key < N ? *reinterpret_cast<const uint32_t*>(src) : 0u;
      }
    }
  };

  auto store_block = [&]() {
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / K_CHUNKS_ROW;
      const int col = ch % K_CHUNKS_ROW;
      *reinterpret_cast<u32x4*>(k_lds + row * KROW + col * 16) = kst[i];
    }
    // V: 4 keys x VD d values -> VD rows of V^T, 4 consecutive keys each.
    uint32_t f16w[4][VD / 2];  // fp16 pairs along d, per key
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int w = 0; w < VD / 2; ++w) {
        if constexpr (ES == 2) {
          f16w[r][w] = v_pair_to_f16<DT, false>(vst[r][w]);
        } else if (w & 1) {
          f16w[r][w] = v_pair_to_f16<DT, true>(vst[r][w / 2]);
        } else {
          f16w[r][w] = v_pair_to_f16<DT, false>(vst[r][w / 2]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < VD; ++e) {
      const int w = e / 2;
      uint32_t lo, hi;
      if (e & 1) {
        lo = (f16w[0][w] >> 16) | (f16w[1][w] & 0xffff0000u);
        hi = (f16w[2][w] >> 16) | (f16w[3][w] & 0xffff0000u);
      } else {
        lo = (f16w[0][w] & 0xffffu) | (f16w[1][w] << 16);
        hi = (f16w[2][w] & 0xffffu) | (f16w[3][w] << 16);
      }
      *reinterpret_cast<u32x2*>(vt_lds + (vc * VD + e) * VROW + 4 * va) = u32x2{lo, hi};
    }
  };

  // ---- running softmax state and the O^T accumulator --------------------------
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};
  float m_run = -INFINITY;  // running max of the raw scores q.k of this query
  float l_run = 0.0f;       // this lane's share of the running row sum

  load_block(0);
  for (int j = 0; j < nblk; ++j) {
    const int kb = j * kBC;
    __syncthreads();  // every wave is done reading the previous block
    store_block();
    __syncthreads();
    if (j + 1 < nblk) load_block(kb + kBC);

    // A wave whose rows all precede this block has nothing to do in it.
    if (CAUSAL && kb > qw0 + kQW - 1) continue;

    // S^T = K_j Q^T: two 32-key tiles of this wave's 32 queries.
    f32x16 st[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      st[kt] = f32x16{};
      const uint8_t* krow = k_lds + (kt * 32 + lr) * KROW;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        QKOperand<DT> a;
        const int byte = (ks * E::kstep + hh * (E::kstep / 2)) * ES;
#pragma unroll
        for (int w = 0; w < E::opnd_dwords; w += 4) {
          u32x4 x = *reinterpret_cast<const u32x4*>(krow + byte + 4 * w);
          a.w[w + 0] = x[0]; a.w[w + 1] = x[1]; a.w[w + 2] = x[2]; a.w[w + 3] = x[3];
        }
        st[kt] = mfma_qk<DT>(a, qreg[ks], st[kt]);
      }
    }

    // Mask keys past N, and (causal) keys after the query.
    const bool need_mask = (kb + kBC > N) || (CAUSAL && kb + kBC - 1 > qw0);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + kt * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
          bool keep = key < N;
          if constexpr (CAUSAL) keep = keep && key <= my_q;
          st[kt][i] = keep ? st[kt][i] : -INFINITY;
        }
      }
    }

    // Online softmax: new running max, rescale factor, probabilities.
    float mx = st[0][0];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = (kt == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, st[kt][i]);
    }
    mx = max_pair32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
    const float mc = m_new * c;
    m_run = m_new;

    float rs = 0.0f;
    uint32_t pw[2][2][4];  // [kt][k-step][dword] fp16 pairs: B operand of O^T += V^T P^T
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(st[kt][i], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(st[kt][i + 1], c, -mc));
        rs += p0 + p1;
        pw[kt][i / 8][(i % 8) / 2] = pack_f16x2(p0, p1);
      }
    }
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int t = 0; t < NDT; ++t) acc[t] *= alpha;

    // O^T += V^T P^T.  Slot j of lane half hh in k-step s of key tile kt holds
    // key kt*32 + 16*s + 8*(j/4) + 4*hh + (j%4), matching the S^T layout.
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      const _Float16* vrow = vt_lds + (t * 32 + lr) * VROW;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int key0 = kt * 32 + 16 * s + 4 * hh;
          u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + key0);
          u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + key0 + 8);
          u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          u32x4 b = {pw[kt][s][0], pw[kt][s][1], pw[kt][s][2], pw[kt][s][3]};
          acc[t] = mfma_pv(a, b, acc[t]);
        }
      }
    }
  }

  // ---- epilogue: O = O^T / l (fp16), LSE = ln 2 * (m*c + log2 l) ---------------
  const float l_tot = sum_pair32(l_run);
  if (my_q < N) {
    const float inv = __builtin_amdgcn_rcpf(l_tot) * v_scale;
    _Float16* orow = p.o + head_off + (int64_t)my_q * D;
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = t * 32 + 8 * g + 4 * hh;
        u32x2 w = {pack_f16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                   pack_f16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    }
    if (hh == 0) {
      p.lse[(int64_t)bh * N + my_q] = kLn2 * (m_run * c + __builtin_amdgcn_logf(l_tot));
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: argument checks (no HIP calls) and launch.
// ---------------------------------------------------------------------------

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
               bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_FP8_E4M3)
    return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) {
    *empty = true;
    return FA_OK;
  }
  // Index arithmetic: rows of one tensor fit in int32, elements in int64;
  // the grid (B*H query-tile rows) fits in int32.
  if (N > (int64_t)1 << 24 || B * H > (int64_t)1 << 24) return FA_ERR_SHAPE;
  const int64_t tiles = (N + kBR - 1) / kBR;
  if (B * H * tiles > INT32_MAX) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  return FA_OK;
}

template <int DT, int D, bool CAUSAL>
int launch_t(const Params& prm, hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&prm)};
  const dim3 grid((unsigned)(prm.bh * prm.n_qtiles));
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_fwd_kernel<DT, D, CAUSAL>),
                                 grid, dim3(kThreads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int DT>
int launch_dt(const Params& prm, int d, int causal, hipStream_t stream) {
  if (d == 64) return causal ? launch_t<DT, 64, true>(prm, stream) : launch_t<DT, 64, false>(prm, stream);
  return causal ? launch_t<DT, 128, true>(prm, stream) : launch_t<DT, 128, false>(prm, stream);
}

int run(const void* q, const void* k, const void* v, const float* dq, const float* dk,
        const float* dv, void* o, float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
        float scale, int causal, int dtype, void* stream) {
  Params prm;
  prm.q = static_cast<const uint8_t*>(q);
  prm.k = static_cast<const uint8_t*>(k);
  prm.v = static_cast<const uint8_t*>(v);
  prm.descale_q = dq;
  prm.descale_k = dk;
  prm.descale_v = dv;
  prm.o = static_cast<_Float16*>(o);
  prm.lse = lse;
  prm.H = (int)H;
  prm.N = (int)N;
  prm.n_qtiles = (int)((N + kBR - 1) / kBR);
  prm.bh = (int)(B * H);
  prm.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case FA_DTYPE_FP16: return launch_dt<FA_DTYPE_FP16>(prm, (int)d, causal, s);
    case FA_DTYPE_BF16: return launch_dt<FA_DTYPE_BF16>(prm, (int)d, causal, s);
    default: return launch_dt<FA_DTYPE_FP8_E4M3>(prm, (int)d, causal, s);
  }
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                      int dtype, void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, &empty);
  if (st != FA_OK || empty) return st;
  return run(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, d, scale, causal, dtype, stream);
}

extern "C" int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* descale_q,
                          const float* descale_k, const float* descale_v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                          void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, FA_DTYPE_FP8_E4M3, &empty);
  if (st != FA_OK || empty) return st;
  if (!descale_q || !descale_k || !descale_v) return FA_ERR_NULL;
  if (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4))
    return FA_ERR_ALIGN;
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal,
             FA_DTYPE_FP8_E4M3, stream);
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is negative or the problem is too large";
    case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case FA_ERR_SCALE: return "scale must be finite and positive";
    case FA_ERR_CAUSAL: return "causal must be 0 or 1";
    default: return "unknown status";
  }
}

extern "C" int fa_abi_version(void) { return FA_ABI_VERSION; }
