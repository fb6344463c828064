// Fused attention backward for MI355X (gfx950, CDNA4): the gradients dQ, dK,
// dV of a loss L, given dO = dL/dO, the inputs Q, K, V, and the forward's O
// and LSE.  The probabilities are recomputed block by block from the saved
// LSE (P_ij = exp(scale q_i.k_j - LSE_i)), so the N x N matrices never reach
// device memory -- the recomputation the "TCA 51%，MFU 不足 8%" page counts
// for the backward pass.  Chain rule through O = P V, P = softmax(S):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = dO_i . O_i,
//   dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernel launches, in this order on the caller's stream:
//   * fa_bwd_dq: one workgroup per (b, h, 256-query tile), a wave per 32
//     queries, shaped like the forward: S^T = K Q^T and dP^T = V dO^T with Q
//     and dO held in registers as B operands, dS^T in registers, then
//     dQ^T += K^T dS^T with K^T read transposed (ds_read_b64_tr_b16) from the
//     row-major K block in LDS; P runs beside the dP matrix instructions and
//     dS beside the dQ ones.  It also computes D_i for its queries from O
//     and dO and stores it (delta), for the second kernel.
//   * fa_bwd_dkdv: one workgroup per (b, h, 128-key tile), two waves per 32
//     keys: a P wave holds the keys' K rows, computes S = Q K^T and P per
//     64-query block, dV^T += dO^T P, and passes P through LDS to the dS wave,
//     which holds the V rows, computes dP = dO V^T, dS = P (dP - D) and
//     dK^T += Q^T dS; dO^T / Q^T are read transposed from the row-major
//     dO / Q blocks.  Each wave's step is a software pipeline: the second
//     product of one block runs beside the elementwise work of the next.
// Blocks stream global -> LDS (buffer_load ... lds, XOR-swizzled 16-byte
// chunks), one barrier per block: the dQ kernel double-buffers K and V and
// unrolls its loop by two (the masked blocks at the end of a wave's range
// run one at a time); the dK/dV kernel keeps four Q stages and two dO stages and
// unrolls by four (running to a multiple of four blocks, the extra blocks
// zero).  Every stage index is thus a constant.  Rows past N read as zeros
// and are masked, as are causal pairs (key j > query i).  P and dS enter the second products
// in the input type (fp16 or bf16, round to nearest even); the dK kernel's dS
// is formed from that rounded P, the dQ kernel's from P in fp32.  All
// accumulation is fp32 and the gradients are stored as fp32.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_common.h"
#include "fa_mi355x.h"

namespace {

constexpr int kBwdWaves = 4;           // key groups of a dK/dV workgroup
constexpr int kRW = 32;                 // rows owned by one wave
constexpr int kBT = kRW * kBwdWaves;    // keys owned by one dK/dV workgroup
constexpr int kDqWaves = 8;             // waves of a dQ workgroup, one per 32 queries
constexpr int kDqThreads = kWave * kDqWaves;
constexpr int kDqT = kRW * kDqWaves;    // queries owned by one dQ workgroup
constexpr int kBS = 64;                 // rows of one streamed block

struct BwdParams {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  const _Float16* o;
  const float* lse;
  const uint8_t* dout;
  float* dq;
  float* dk;
  float* dv;
  float* delta;
  int N;
  int n_tiles;
  int bh;
  int n_xcd;  // XCDs of the device (workgroup -> XCD mapping of tile_of)
  float scale;
};

template <int DT>
__device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == FA_DTYPE_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return mfma_pv(a, b, c);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats as a pair of the input type, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (DT == FA_DTYPE_BF16) {
    bf16x2 h = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, h);
  } else {
    return pack_f16x2(lo, hi);
  }
}

// Element e (0 or 1) of a pair of the input type, as float (exact).
template <int DT>
__device__ __forceinline__ float elem(uint32_t w, int e) {
  const uint32_t bits = e ? (w >> 16) : (w & 0xffffu);
  if constexpr (DT == FA_DTYPE_BF16) {
    return __uint_as_float(bits << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  }
}

typedef __attribute__((address_space(3))) short4_t lds_short4_t_bwd;

// Per-lane addresses into a row-major LDS block of ROWB-byte rows whose
// 16-byte chunks carry the swizzle swz<ROWB>(row):
//  * row operand (A of a 32x32x16 MFMA with rows as M): row r0 + lr, the 8
//    d-values of k-step ks starting at ks*16 + 8*hh;
//  * transposed operand (A with d as M and rows as the contraction): lane
//    (grp, e, r) of each 16-lane group reads 4 d-values of one row; the
//    transposing read hands each lane the 4 rows at its d-value.  Slot j of
//    lane half hh in k-step s is row 16 s + 8 (j / 4) + 4 hh + (j % 4) --
//    the order a 32x32 accumulator holds its rows, so the other operand can
//    come straight from an accumulator.
template <int ROWB>
struct BlockAddr {
  static constexpr int D = ROWB / 2;
  static constexpr int NKS = D / 16;
  static constexpr int NDT = D / 32;
  int row[NKS];        // + tile_row * ROWB
  int tr[NDT][2];      // + (16-row group) * ROWB
  __device__ __forceinline__ void init(int lane) {
    const int lr = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int chunk = (ks * 16 + 8 * hh) / 8;
      row[ks] = lr * ROWB + ((chunk ^ swz<ROWB>(lr)) * 16);
    }
    const int grp = lane >> 4, li = lane & 15, e = li >> 2, r = li & 3;
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int rr = 8 * half + 4 * (grp >> 1) + e;
        const int d = t * 32 + 16 * (grp & 1) + 4 * r;
        tr[t][half] = rr * ROWB + (((d / 8) ^ swz<ROWB>(rr)) * 16) + (d % 8) * 2;
      }
  }
};

// A operand (32 rows x 16 d-values at k-step ks) of rows tile_row*32 .. +31.
template <int ROWB>
__device__ __forceinline__ u32x4 row_operand(const uint8_t* blk, const BlockAddr<ROWB>& a,
                                             int tile, int ks) {
  return *reinterpret_cast<const u32x4*>(blk + tile * 32 * ROWB + a.row[ks]);
}

// A operand (32 d-values of d tile t x 16 rows 16*g .. +15, in accumulator
// row order) read transposed from the row-major block.
template <int ROWB>
__device__ __forceinline__ u32x4 tr_operand(const uint8_t* blk, const BlockAddr<ROWB>& a, int t,
                                            int g) {
  const uint8_t* base = blk + g * 16 * ROWB;
  short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t_bwd*)(base + a.tr[t][0]));
  short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t_bwd*)(base + a.tr[t][1]));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  return u32x4{l2[0], l2[1], h2[0], h2[1]};
}

// Streams 64-row blocks of one head's [N, D] tensor into LDS: block rows
// land at row * ROWB with swizzled chunks; one 64-lane load instruction fills
// 1 KB, the workgroup's waves share the instructions.  Rows at or past N,
// and blocks past `end_row`, read zeros (the latter without memory traffic).
template <int ROWB, int W = kBwdWaves>
struct BlockLoader {
  static constexpr int CPR = ROWB / 16;
  static constexpr int INSTR = kBS * CPR / kWave;
  static_assert(INSTR % W == 0, "block must split evenly over the waves");
  static constexpr int PER_W = INSTR / W;
  int goff[PER_W];
  int wave;
  __device__ __forceinline__ void init(int w, int lane) {
    wave = w;
#pragma unroll
    for (int u = 0; u < PER_W; ++u) {
      const int slot = (u * W + w) * kWave + lane;
      const int row = slot / CPR, phys = slot % CPR;
      goff[u] = row * ROWB + ((phys ^ swz<ROWB>(row)) * 16);
    }
  }
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, uint8_t* blk, int row0,
                                       int end_row) const {
    const int boff = row0 < end_row ? row0 * ROWB : (1 << 30);
#pragma unroll
    for (int u = 0; u < PER_W; ++u)
      buffer_to_lds16(rs, blk + (u * W + wave) * kWave * 16, goff[u] + boff, 0);
  }
};

// 4 bytes per lane from a buffer straight into LDS: lane t writes
// lds_dst + 4 t; each lane's dword is range-checked on its own.
__device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t rs, void* lds_dst,
                                               int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)lds_dst, 4, voffset, 0, 0, 0);
}

// Stores one wave's 32 x D fp32 block -- accumulators in the 32x32 MFMA
// layout (lane l: row l % 32, d values t*32 + 8*(i/4) + 4*(l/32) + i%4 of
// acc[t][i]), times f -- as whole rows: through the wave's own LDS region buf
// (32 * D * 4 bytes, 16-byte chunks XOR-swizzled by row), read back
// row-major, 16 bytes per lane.  Stored straight from the accumulators, each
// instruction would scatter 16-byte pieces over 32 rows, and a wave retires
// only once its stores have completed.  rows: row 0 of the block in global
// memory (rows D floats apart); rows at or past n_rows are not stored.
template <int D>
__device__ __forceinline__ void store_rows_f32(const f32x16* acc, float f, uint8_t* buf,
                                               float* rows, int n_rows, int lane) {
  constexpr int ROWB = D * 4;      // bytes of one row
  constexpr int CH = ROWB / 16;    // 16-byte chunks per row
  constexpr int RPI = kWave / CH;  // rows per read instruction
  const int lr = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ch = 8 * t + 2 * g + hh;  // d values 4 * ch .. +3
      *reinterpret_cast<f32x4*>(buf + lr * ROWB + ((ch ^ (lr % CH)) * 16)) =
          f32x4{acc[t][4 * g] * f, acc[t][4 * g + 1] * f, acc[t][4 * g + 2] * f,
                acc[t][4 * g + 3] * f};
    }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int it = 0; it < 32 / RPI; ++it) {
    const int r = it * RPI + lane / CH, ch = lane % CH;
    const f32x4 x = *reinterpret_cast<const f32x4*>(buf + r * ROWB + ((ch ^ (r % CH)) * 16));
    if (r < n_rows) *reinterpret_cast<f32x4*>(rows + (int64_t)r * D + ch * 4) = x;
  }
}

__device__ __forceinline__ void bwd_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// dQ (and D = rowsum(dO * O)).
// ---------------------------------------------------------------------------
// Slices of the dQ step.  The run is S (chain of accumulator 0, then 1),
// dP (likewise), then dQ in four groups of NDT matrix instructions, group
// G = (t2, sg) taking dS elements 8 sg .. 8 sg + 7 of accumulator t2.
// dq_vp(i): slice of element i's (0 .. 31; accumulator i / 16) P: its FMA,
// the exponential one slice later (and, in a masked block, the mask one
// later still), once S's chain has completed.  dq_vd(i): slice of its dS:
// the subtraction, the product one slice later, the pack of a pair two
// slices later -- after dP's chain has completed and before its group's
// matrix instructions.
template <int NKS, int NDT>
constexpr int dq_vp(int i) {
  constexpr int NS = 2 * NKS;
  return i < 16 ? NKS + 1 + (i * (NS - 1)) / 16 : NS + 1 + ((i - 16) * (NS - 1)) / 16;
}
template <int NKS, int NDT>
constexpr int dq_vd(int i) {
  constexpr int NS = 2 * NKS;
  const int t2 = i / 16, e = i % 16, g = 2 * t2 + e / 8;
  const int ready = t2 == 0 ? NS + NKS + 1 : 2 * NS + 1;
  const int last = 2 * NS + g * NDT - 3;
  const int first = ready > last - 4 ? ready : last - 4;
  return first + ((e % 8) * (last - first + 1)) / 8;
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kDqThreads, 1) void fa_bwd_dq_kernel(BwdParams p) {
  constexpr int ROWB = D * 2;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int BLK = kBS * ROWB;
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[BLK];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds1[BLK];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds0[BLK];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds1[BLK];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 31, hh = lane >> 5;

  int bh, qt;
  tile_of(blockIdx.x, p.bh, p.n_tiles, CAUSAL, p.n_xcd, bh, qt);
  const int N = p.N;
  const int64_t head_off = (int64_t)bh * N * D;
  const int head_bytes = N * ROWB;
  const __amdgpu_buffer_rsrc_t qrs = head_rsrc(p.q + head_off * 2, head_bytes);
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(p.k + head_off * 2, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(p.v + head_off * 2, head_bytes);
  const __amdgpu_buffer_rsrc_t ors = head_rsrc(
      reinterpret_cast<const uint8_t*>(p.o + head_off), head_bytes);
  const __amdgpu_buffer_rsrc_t dors = head_rsrc(p.dout + head_off * 2, head_bytes);

  const int q0 = qt * kDqT;
  const int qw0 = q0 + wave * kRW;  // first query of this wave
  const int my_q = qw0 + lr;
  const float cs = p.scale * kLog2e;

  // Q and dO rows of this lane's query (B operands), and D = dO . O.
  u32x4 qreg[NKS], doreg[NKS];
  float dpart = 0.0f;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int byte = my_q * ROWB + (ks * 16 + 8 * hh) * 2;
    qreg[ks] = __builtin_amdgcn_raw_buffer_load_b128(qrs, byte, 0, 0);
    doreg[ks] = __builtin_amdgcn_raw_buffer_load_b128(dors, byte, 0, 0);
    const u32x4 ow = __builtin_amdgcn_raw_buffer_load_b128(ors, byte, 0, 0);
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        dpart = fmaf(elem<DT>(doreg[ks][w], e), elem<FA_DTYPE_FP16>(ow[w], e), dpart);
  }
  const float dsum = sum_pair32(dpart);
  const float lse_l2 = (my_q < N ? p.lse[(int64_t)bh * N + my_q] : 0.0f) * kLog2e;
  if (hh == 0 && my_q < N) p.delta[(int64_t)bh * N + my_q] = dsum;

  BlockAddr<ROWB> ka;
  ka.init(lane);
  BlockLoader<ROWB, kDqWaves> ld;
  ld.init(wave, lane);

  int kv_end = N;
  if constexpr (CAUSAL) kv_end = min(N, q0 + kDqT);
  const int nblk = (kv_end + kBS - 1) / kBS;

  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};

  ld.load(krs, k_lds0, 0, kv_end);
  ld.load(vrs, v_lds0, 0, kv_end);
  bwd_barrier();

  // One step (key block j) as a software pipeline of NM slices: slice m
  // issues matrix instruction m, the LDS operand reads of instruction
  // m + LA, and its share of the elementwise work (dq_vp, dq_vd), so that
  // P = exp2(cs S - LSE log2 e) runs beside the dP instructions and dS^T =
  // P^T (dP^T - D) beside the dQ instructions of the group before.  A
  // scheduling barrier closes every slice.  MASKED: the block reaches past N
  // or, causal, past this wave's first query; its masked pairs get P = 0.
  constexpr int NS = 2 * NKS;
  constexpr int NM = 2 * NS + 4 * NDT;
  constexpr int LA = 2;
  static_assert(dq_vd<NKS, NDT>(31) + 2 < NM, "slice plan out of range");
  auto step = [&](int j, const uint8_t* kb, const uint8_t* vb, uint8_t* kn, uint8_t* vn,
                  auto mc) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(mc)::value;
    ld.load(krs, kn, (j + 1) * kBS, kv_end);  // next block, in flight during this one
    ld.load(vrs, vn, (j + 1) * kBS, kv_end);
    const int kb0 = j * kBS;
    f32x16 st[2], dpt[2];
    u32x4 opnd[LA];
    uint32_t dsw[2][2][4];
    auto read = [&](auto rc) __attribute__((always_inline)) {
      constexpr int m = decltype(rc)::value;
      if constexpr (m < 2 * NS) {
        opnd[m % LA] = row_operand<ROWB>(m < NS ? kb : vb, ka, (m % NS) / NKS, m % NKS);
      } else {
        constexpr int q = m - 2 * NS, g = q / NDT, t = q % NDT;
        opnd[m % LA] = tr_operand<ROWB>(kb, ka, t, g);
      }
    };
    auto mfma = [&](auto rc) __attribute__((always_inline)) {
      constexpr int m = decltype(rc)::value;
      if constexpr (m < NS) {
        constexpr int t2 = m / NKS, ks = m % NKS;
        st[t2] = mfma16<DT>(opnd[m % LA], qreg[ks], ks == 0 ? f32x16{} : st[t2]);
      } else if constexpr (m < 2 * NS) {
        constexpr int t2 = (m - NS) / NKS, ks = (m - NS) % NKS;
        dpt[t2] = mfma16<DT>(opnd[m % LA], doreg[ks], ks == 0 ? f32x16{} : dpt[t2]);
      } else {
        constexpr int q = m - 2 * NS, g = q / NDT, t = q % NDT;
        const u32x4 b = {dsw[g / 2][g % 2][0], dsw[g / 2][g % 2][1], dsw[g / 2][g % 2][2],
                         dsw[g / 2][g % 2][3]};
        acc[t] = mfma16<DT>(opnd[m % LA], b, acc[t]);
      }
    };
    auto elementwise = [&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int t2 = i / 16, e = i % 16;
        const int vp = dq_vp<NKS, NDT>(i), vd = dq_vd<NKS, NDT>(i);
        if (vp == k) st[t2][e] = fmaf(st[t2][e], cs, -lse_l2);
        if (vp + 1 == k) st[t2][e] = __builtin_amdgcn_exp2f(st[t2][e]);
        if (MASKED && vp + 2 == k) {
          const int key = kb0 + t2 * 32 + 8 * (e / 4) + 4 * hh + (e % 4);
          bool keep = key < N;
          if constexpr (CAUSAL) keep = keep && key <= my_q;
          st[t2][e] = keep ? st[t2][e] : 0.0f;
        }
        if (vd == k) dpt[t2][e] -= dsum;
        if (vd + 1 == k) dpt[t2][e] *= st[t2][e];
        if (i % 2 == 1 && vd + 2 == k)
          dsw[t2][e / 8][(e % 8) / 2] = pack2<DT>(dpt[t2][e - 1], dpt[t2][e]);
      }
    };
    static_for<0, LA>(read);
    __builtin_amdgcn_sched_barrier(0);
    static_for<0, NM>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      mfma(kc);
      if constexpr (k + LA < NM) read(std::integral_constant<int, k + LA>{});
      elementwise(kc);
      __builtin_amdgcn_sched_barrier(0);
    });
    bwd_barrier();
  };
  // Only a block reaching past N or past the wave's first query needs the
  // mask, and those blocks end the wave's range: blocks from j_edge on.  The
  // loop runs the plain step in pairs (stage indices fixed per copy) below
  // j_edge, then the masked step, stages chosen at run time, to the end.
  // Every wave passes nblk barriers.
  using Plain = std::false_type;
  using Masked = std::true_type;
  int j_edge = min(nblk, N / kBS);
  if constexpr (CAUSAL) j_edge = min(j_edge, qw0 / kBS);
  int j = 0;
  for (; j + 2 <= j_edge; j += 2) {
    step(j, k_lds0, v_lds0, k_lds1, v_lds1, Plain{});
    step(j + 1, k_lds1, v_lds1, k_lds0, v_lds0, Plain{});
  }
  for (; j < nblk; ++j) {
    const bool odd = j & 1;
    step(j, odd ? k_lds1 : k_lds0, odd ? v_lds1 : v_lds0, odd ? k_lds0 : k_lds1,
         odd ? v_lds0 : v_lds1, Masked{});
  }

  // The loop's last barrier has drained every load and LDS access: the K and
  // V stages (one 32 x D fp32 block each) are free for the row-wise store,
  // four waves at a time.
  static_assert(kDqWaves == 8 && BLK == kRW * D * 4, "one 32 x D fp32 block per stage");
  const int sw = wave % 4;
  uint8_t* sbuf = sw == 0 ? k_lds0 : sw == 1 ? k_lds1 : sw == 2 ? v_lds0 : v_lds1;
  float* dq_rows = p.dq + head_off + (int64_t)qw0 * D;
  if (wave < 4) store_rows_f32<D>(acc, p.scale, sbuf, dq_rows, N - qw0, lane);
  __syncthreads();
  if (wave >= 4) store_rows_f32<D>(acc, p.scale, sbuf, dq_rows, N - qw0, lane);
}

// ---------------------------------------------------------------------------
// dK and dV in one pass over the query blocks, by two kinds of wave per
// 32-key group: the P wave computes S = Q K^T, P and dV^T += dO^T P, and hands
// P (in the input type) to the group's dS wave through LDS; the dS wave
// computes dP = dO V^T, dS = P (dP - D) and dK^T += Q^T dS.  Four products per
// block, where a dV pass and a dK pass of their own would take five (S twice);
// each wave holds one key operand and one accumulator, so all eight fit two
// waves per SIMD (one of each kind), and each kind's elementwise work issues
// beside the matrix instructions of its own second product and of the other
// kind's wave on the SIMD.
// ---------------------------------------------------------------------------
constexpr int kKVWaves = 2 * kBwdWaves;  // waves 0-3: P, 4-7: dS, of key group wave % 4
constexpr int kKVThreads = kWave * kKVWaves;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Slice of the dK/dV step in which element e (0 .. 31; accumulator e / 16,
// element e % 16) of the first product gets its first elementwise operation.
// The run is 2 NKS first-product matrix instructions, accumulator 0's chain
// first, then NM - 2 NKS second-product ones: accumulator 0's elements start
// two slices after its chain's last instruction, accumulator 1's likewise, and
// the last element leaves two slices for its remaining operations.
template <int NKS, int NM>
constexpr int bwd_vslice(int e) {
  constexpr int R0 = NKS + 1, R1 = 2 * NKS + 1, RL = NM - 2;
  return e < 16 ? R0 + (e * (R1 - R0)) / 16 : R1 + ((e - 16) * (RL - R1 + 1)) / 16;
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kKVThreads, 1) void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int ROWB = D * 2;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int BLK = kBS * ROWB;
  constexpr int PBLK = kRW * kBS * 2;  // one group's P block in the input type
  // Step j of the loop, in each 32-key group:
  //   P wave:  S(j+1) = Q(j+1) K^T, then dV^T += dO(j)^T P(j) with P(j) in
  //            registers since step j-1, while the exponentials of S(j+1)
  //            run beside those matrix instructions; P(j+1) goes to LDS.
  //   dS wave: dP(j) = dO(j) V^T, then dK^T += Q(j-1)^T dS(j-1) with dS(j-1)
  //            in registers since step j-1, while dS(j) = P(j) (dP(j) - D(j))
  //            is formed beside them from the P(j) its P wave stored.
  // Meanwhile Q(j+2) and dO(j+1) stream in.  Q is read as Q(j+1) and Q(j-1)
  // and loaded as Q(j+2): four stages; dO, P, LSE and D two each.  One
  // barrier a step.
  //
  // LDS, one buffer: Q stages, dO stages, P (per stage and key group: lane
  // l's 16 dwords as four 16-byte pieces at (c * 64 + l) * 16, c = 0 .. 3),
  // LSE (times log2 e; +inf for rows at or past N) and D of a block's 64
  // queries.  Every access in the loop is a per-lane base register plus an
  // immediate offset (16 bits): each wave keeps one base into the Q or dO
  // stages for its row-wise reads and one into the other for its transposed
  // reads, so no stage needs registers of its own.
  constexpr int OFF_Q = 0;
  constexpr int OFF_DO = OFF_Q + 4 * BLK;
  constexpr int OFF_P = OFF_DO + 2 * BLK;
  constexpr int PSTAGE = kBwdWaves * PBLK;
  constexpr int OFF_LSE = OFF_P + 2 * PSTAGE;
  constexpr int OFF_D = OFF_LSE + 2 * kBS * 4;
  constexpr int LDS_BYTES = OFF_D + 2 * kBS * 4;
  static_assert(3 * BLK + 3 * 16 * ROWB <= 65535 && PSTAGE + 3 * 1024 <= 65535,
                "immediate offsets must fit 16 bits");
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int hh = lane >> 5;
  const bool pw = wave < kBwdWaves;  // P wave, else dS wave (wave-uniform)
  const int grp = wave % kBwdWaves;

  // Causal work shrinks with the key tile: tile_of hands out its heavy-first
  // order in reverse tile index, so turn it around.
  int bh, tt;
  tile_of(blockIdx.x, p.bh, p.n_tiles, CAUSAL, p.n_xcd, bh, tt);
  const int kt = CAUSAL ? p.n_tiles - 1 - tt : tt;
  const int N = p.N;
  const int64_t head_off = (int64_t)bh * N * D;
  const int head_bytes = N * ROWB;
  const __amdgpu_buffer_rsrc_t qrs = head_rsrc(p.q + head_off * 2, head_bytes);
  const __amdgpu_buffer_rsrc_t kvrs = head_rsrc((pw ? p.k : p.v) + head_off * 2, head_bytes);
  const __amdgpu_buffer_rsrc_t dors = head_rsrc(p.dout + head_off * 2, head_bytes);
  const __amdgpu_buffer_rsrc_t lrs = head_rsrc(
      reinterpret_cast<const uint8_t*>(p.lse + (int64_t)bh * N), N * 4);
  const __amdgpu_buffer_rsrc_t drs = head_rsrc(
      reinterpret_cast<const uint8_t*>(p.delta + (int64_t)bh * N), N * 4);

  const int k0 = kt * kBT;
  const int my_k = k0 + grp * kRW + (lane & 31);
  const float cs = p.scale * kLog2e;

  // This lane's key row of K (P wave) or V (dS wave): the B operand of
  // S = Q K^T or dP = dO V^T.
  u32x4 kv[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kv[ks] = __builtin_amdgcn_raw_buffer_load_b128(kvrs, my_k * ROWB + (ks * 16 + 8 * hh) * 2, 0, 0);
  // The dS wave holds -V: its product, started from D instead of zero,
  // accumulates D - dP, and dS = P (dP - D) = (-P) (D - dP) needs no
  // subtraction (the sign is a free source modifier of the multiply).
  if (!pw) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kv[ks] ^= 0x80008000u;
  }

  BlockAddr<ROWB> qa;
  qa.init(lane);
  BlockLoader<ROWB, kKVWaves> ld;
  ld.init(wave, lane);
  // Per-lane LDS bases (opaque to the compiler, so that it keeps one register
  // each instead of one per stage): row-wise reads of the first product's A
  // block (Q for a P wave, dO for a dS wave), transposed reads of the second
  // product's block (dO, Q), this lane's P pieces, and the per-row values
  // (LSE for a P wave, D for a dS wave) at this lane's half.
  uint32_t arow[NKS], atr[NDT][2];
  const uint32_t a_win = pw ? OFF_Q : OFF_DO, t_win = pw ? OFF_DO : OFF_Q;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    arow[ks] = qa.row[ks] + a_win;
    asm volatile("" : "+v"(arow[ks]));
  }
#pragma unroll
  for (int t = 0; t < NDT; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      atr[t][h] = qa.tr[t][h] + t_win;
      asm volatile("" : "+v"(atr[t][h]));
    }
  uint32_t pbase = OFF_P + grp * PBLK + lane * 16;
  uint32_t rbase = (pw ? OFF_LSE : OFF_D) + 16 * hh;
  asm volatile("" : "+v"(pbase), "+v"(rbase));
  auto lds16 = [&](uint32_t base, int off) __attribute__((always_inline)) {
    return *reinterpret_cast<const u32x4*>(smem + base + off);
  };
  // A operand at row tile t2, k-step ks of the block at byte `stage` of the
  // A window; transposed operand (d tile t, 16-row group g) likewise.
  auto a_read = [&](int stage, int t2, int ks) __attribute__((always_inline)) {
    return lds16(arow[ks], stage + t2 * 32 * ROWB);
  };
  auto t_read = [&](int stage, int t, int g) __attribute__((always_inline)) {
    const int off = stage + g * 16 * ROWB;
    short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4_t_bwd*)(smem + atr[t][0] + off));
    short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_short4_t_bwd*)(smem + atr[t][1] + off));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  };

  // Query blocks that can see a key of this tile: all, or (causal) from the
  // block holding query k0 on.
  const int qb_begin = CAUSAL ? (k0 / kBS) : 0;
  const int nblk = (N - qb_begin * kBS + kBS - 1) / kBS;
  auto row0_of = [&](int j) { return (qb_begin + j) * kBS; };

  f32x16 acc[NDT];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};

  // LSE and D rows of a block, one dword per lane: D goes straight to LDS
  // (wave 1); LSE passes through wave 0's registers to be stored already
  // multiplied by log2 e, once per row instead of once per score.  A row at
  // or past N stores +inf, so that its probabilities come out 0 without a
  // mask.
  float lse_next = 0.0f;
  auto load_lse = [&](int row0) __attribute__((always_inline)) {
    const int off = (row0 < N ? row0 : N) * 4 + lane * 4;  // past N: zeros
    if (wave == 0) lse_next = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, off, 0, 0));
  };
  auto store_lse = [&](int stage, int row0) __attribute__((always_inline)) {
    if (wave == 0)
      reinterpret_cast<float*>(smem + OFF_LSE + stage * kBS * 4)[lane] =
          row0 + lane < N ? lse_next * kLog2e : __builtin_inff();
  };
  auto load_d = [&](int stage, int row0) __attribute__((always_inline)) {
    const int off = (row0 < N ? row0 : N) * 4 + lane * 4;
    if (wave == 1) buffer_to_lds4(drs, smem + OFF_D + stage * kBS * 4, off);
  };
  auto load_q = [&](int stage, int row0) __attribute__((always_inline)) {
    ld.load(qrs, smem + OFF_Q + stage * BLK, row0, N);
  };
  auto load_do = [&](int stage, int row0) __attribute__((always_inline)) {
    ld.load(dors, smem + OFF_DO + stage * BLK, row0, N);
  };

  // Element e (0 .. 15) of accumulator t2 is query row t2*32 + 8*(e/4) +
  // 4*hh + e%4 of the block; its pair (e, e+1), e even, is dword
  // w[t2][e/8][(e%8)/2] of the block's P or dS registers -- the order in which
  // the 32x32 MFMA takes its B operand for the second products.
  using BRegs = uint32_t[2][2][4];
  auto brow = [&](int t2, int e) { return t2 * 32 + 8 * (e / 4) + 4 * hh + e % 4; };
  // Zeroes the probabilities of causally masked pairs (query before key) in
  // the block starting at query qrow0.
  auto causal_mask = [&](BRegs& w, int qrow0) __attribute__((always_inline)) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const int qi = qrow0 + brow(t2, e);  // rows qi, qi + 1
        const uint32_t m = (qi >= my_k ? 0xffffu : 0u) | (qi + 1 >= my_k ? 0xffff0000u : 0u);
        w[t2][e / 8][(e % 8) / 2] &= m;
      }
  };
  auto store_b = [&](int stage, const BRegs& w) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4*>(smem + pbase + stage * PSTAGE + c * kWave * 16) =
          u32x4{w[c / 2][c % 2][0], w[c / 2][c % 2][1], w[c / 2][c % 2][2], w[c / 2][c % 2][3]};
  };
  auto load_b = [&](int stage, BRegs& w) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 pv = lds16(pbase, stage * PSTAGE + c * kWave * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[c / 2][c % 2][e] = pv[e];
    }
  };

  // Block 0's P (P waves), before the loop: S = Q K^T, then P with the
  // causal mask, to LDS and into w.
  auto first_p = [&](BRegs& w) __attribute__((always_inline)) {
    f32x16 x[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) x[t2] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) x[t2] = mfma16<DT>(a_read(0, t2, ks), kv[ks], x[t2]);
    mfma_read_pipeline<2 * NKS, 1, 4>();
    __builtin_amdgcn_sched_barrier(0);
    const float* lb = reinterpret_cast<const float*>(smem + OFF_LSE);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        float pt[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          pt[i] = __builtin_amdgcn_exp2f(fmaf(x[t2][e + i], cs, -lb[brow(t2, e + i)]));
          if (CAUSAL && row0_of(0) + brow(t2, e + i) < my_k) pt[i] = 0.0f;
        }
        w[t2][e / 8][(e % 8) / 2] = pack2<DT>(pt[0], pt[1]);
      }
    store_b(0, w);
  };

  // Q stage 3 stands for the block before block 0 in the dK product of step
  // 0 (against a zero dS): zero it, as uninitialised LDS may hold NaNs.
  for (int i = tid; i < BLK / 16; i += kKVThreads)
    reinterpret_cast<u32x4*>(smem + OFF_Q + 3 * BLK)[i] = u32x4{0u, 0u, 0u, 0u};
  load_q(0, row0_of(0));
  load_q(1, row0_of(1));
  load_do(0, row0_of(0));
  load_d(0, row0_of(0));
  load_lse(row0_of(0));
  store_lse(0, row0_of(0));
  load_lse(row0_of(1));
  store_lse(1, row0_of(1));
  bwd_barrier();
  // Registers ra / rb: P(j) and P(j+1) of a P wave, dS(j-1) and dS(j) of a dS
  // wave, alternating with the step's parity; dS(-1) is zero.
  uint32_t ra[2][2][4], rb[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c) ra[a][b][c] = rb[a][b][c] = 0u;
  if (pw) first_p(ra);
  bwd_barrier();

  // One step as a software pipeline of NM slices, like the forward's: slice m
  // issues matrix instruction m (the 2 NKS of the first product, chain of
  // accumulator t2 = 0 first, then the 4 NDT of the second), the LDS operand
  // reads of instruction m + LA, and its share of the elementwise work on the
  // first product's result: element e's first operation in slice
  // bwd_vslice(e), once its accumulator's chain has completed, the second one
  // slice later, the pack of a pair two slices later.  A scheduling barrier
  // closes every slice.
  constexpr int NS = 2 * NKS;
  constexpr int NM = NS + 4 * NDT;
  constexpr int LA = 4;
  static_assert(bwd_vslice<NKS, NM>(0) - 3 >= 0 && bwd_vslice<NKS, NM>(31) + 2 <= NM,
                "slice plan out of range");

  // Each kind of wave runs its own copy of the loop (PW: the kind, a
  // compile-time constant inside); both copies meet at the same barriers.
  auto main_loop = [&](auto pwc) __attribute__((always_inline)) {
    constexpr bool PW = decltype(pwc)::value;
    auto step = [&](int j, auto uc, BRegs& r_prev, BRegs& r_cur) __attribute__((always_inline)) {
      constexpr int U = decltype(uc)::value;
      // Stages: Q(j+1) at (U+1)%4, Q(j-1) at (U+3)%4, Q(j+2) loads into
      // (U+2)%4; dO(j), D(j), P(j) at U%2; LSE(j+1) at (U+1)%2.  Offsets of
      // the stages within the A and transposed windows, and of the per-row
      // values (LSE(j+1) log2 e or D(j)):
      constexpr int QP = (U + 1) % 4, QD = (U + 3) % 4, QL = (U + 2) % 4;
      constexpr int S0 = U % 2, S1 = (U + 1) % 2;
      constexpr int AS = PW ? QP * BLK : S0 * BLK;
      constexpr int TS = PW ? S0 * BLK : QD * BLK;
      constexpr int RS = (PW ? S1 : S0) * kBS * 4;
      load_q(QL, row0_of(j + 2));
      load_do(S1, row0_of(j + 1));
      load_d(S1, row0_of(j + 1));
      load_lse(row0_of(j + 2));
      f32x16 x[2];
      u32x4 opnd[LA];
      f32x4 r4[2][4];
      auto read = [&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m < NS) {
          opnd[m % LA] = a_read(AS, m / NKS, m % NKS);
        } else {
          constexpr int q = m - NS, t2 = q / (2 * NDT), sg = (q / NDT) % 2, t = q % NDT;
          opnd[m % LA] = t_read(TS, t, 2 * t2 + sg);
        }
      };
      auto mfma = [&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m < NS) {
          constexpr int t2 = m / NKS, ks = m % NKS;
          f32x16 c = x[t2];
          if constexpr (ks == 0) {
            if constexpr (PW) {
              c = f32x16{};
            } else {
#pragma unroll
              for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i) c[4 * g + i] = r4[t2][g][i];  // D of the rows
            }
          }
          x[t2] = mfma16<DT>(opnd[m % LA], kv[ks], c);
        } else {
          constexpr int q = m - NS, t2 = q / (2 * NDT), sg = (q / NDT) % 2, t = q % NDT;
          const u32x4 b = {r_prev[t2][sg][0], r_prev[t2][sg][1], r_prev[t2][sg][2],
                           r_prev[t2][sg][3]};
          acc[t] = mfma16<DT>(opnd[m % LA], b, acc[t]);
        }
      };
      // The per-row values of accumulator t2: four 16-byte reads.
      auto read_r4 = [&](int t2) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          r4[t2][g] = __builtin_bit_cast(f32x4, lds16(rbase, RS + t2 * 32 * 4 + 8 * g * 4));
      };
      // P wave: P = exp2(S cs - LSE log2 e), packed into r_cur.
      // dS wave: dS = (-P) (D - dP), P read from r_cur, packed back into it.
      auto elementwise = [&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (PW) {
#pragma unroll
          for (int g = 0; g < 8; ++g)
            if (bwd_vslice<NKS, NM>(4 * g) - 3 == k)
              r4[g / 4][g % 4] = __builtin_bit_cast(
                  f32x4, lds16(rbase, RS + (g / 4) * 32 * 4 + 8 * (g % 4) * 4));
        } else {
          if constexpr (k == NKS / 2) read_r4(1);  // D for accumulator 1's chain
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int t2 = i / 16, e = i % 16, v0 = bwd_vslice<NKS, NM>(i);
          if constexpr (PW) {
            if (v0 == k) x[t2][e] = fmaf(x[t2][e], cs, -r4[t2][e / 4][e % 4]);
            if (v0 + 1 == k) x[t2][e] = __builtin_amdgcn_exp2f(x[t2][e]);
          } else {
            if (v0 + 1 == k) x[t2][e] *= -elem<DT>(r_cur[t2][e / 8][(e % 8) / 2], e % 2);
          }
          if (i % 2 == 1 && v0 + 2 == k)
            r_cur[t2][e / 8][(e % 8) / 2] = pack2<DT>(x[t2][e - 1], x[t2][e]);
        }
      };
      if constexpr (!PW) read_r4(0);  // D for accumulator 0's chain
      static_for<0, LA>(read);
      if constexpr (!PW) load_b(S0, r_cur);  // P(j)
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NM + 1>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < NM) mfma(kc);
        if constexpr (k + LA < NM) read(std::integral_constant<int, k + LA>{});
        elementwise(kc);
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (PW) {
        // Only S(1) of the loop's blocks can hold causally masked pairs.
        if constexpr (CAUSAL && U == 0)
          if (j == 0) causal_mask(r_cur, row0_of(1));
        store_b(S1, r_cur);  // P(j+1)
      } else {
        // dS(j) is first used by the next step's matrix instructions: without
        // this use here the compiler sinks its computation past the barrier,
        // out of the slices it was meant to share.
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int c = 0; c < 4; ++c) asm volatile("" ::"v"(r_cur[a][b][c]));
      }
      store_lse(S0, row0_of(j + 2));  // stage S0 held LSE(j), last used in step j-1
      bwd_barrier();
    };
    // After the last step (block j), a dS wave still owes dK^T += Q(j)^T dS(j).
    auto last = [&](auto uc, const BRegs& w) __attribute__((always_inline)) {
      constexpr int U = decltype(uc)::value;
      if constexpr (!PW) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int sg = 0; sg < 2; ++sg)
#pragma unroll
            for (int t = 0; t < NDT; ++t) {
              const u32x4 b = {w[t2][sg][0], w[t2][sg][1], w[t2][sg][2], w[t2][sg][3]};
              acc[t] = mfma16<DT>(t_read((U % 4) * BLK, t, 2 * t2 + sg), b, acc[t]);
            }
        mfma_read_pipeline<4 * NDT, 2, 4>();
      }
    };
    // Four steps per trip (stage indices fixed per copy), to the next multiple
    // of four blocks: blocks past the last one load as zeros with LSE +inf,
    // so their P and dS are 0 and they change neither dV nor dK.
    for (int j = 0; j < nblk; j += 4) {
      step(j, std::integral_constant<int, 0>{}, ra, rb);
      step(j + 1, std::integral_constant<int, 1>{}, rb, ra);
      step(j + 2, std::integral_constant<int, 2>{}, ra, rb);
      step(j + 3, std::integral_constant<int, 3>{}, rb, ra);
    }
    last(std::integral_constant<int, 3>{}, ra);
  };
  if (pw)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});

  // dV leaves through the dO and P stages (the dS waves may still read a Q
  // stage for their last product), then dK through the Q stages.
  static_assert(kBwdWaves == 4 && BLK == kRW * D * 4 && 2 * PSTAGE >= 2 * BLK,
                "one 32 x D fp32 block per stage");
  const int kw0 = k0 + grp * kRW;
  if (pw) {
    uint8_t* sbuf = smem + (grp < 2 ? OFF_DO + grp * BLK : OFF_P + (grp - 2) * BLK);
    store_rows_f32<D>(acc, 1.0f, sbuf, p.dv + head_off + (int64_t)kw0 * D, N - kw0, lane);
  }
  lds_barrier();
  if (!pw)
    store_rows_f32<D>(acc, p.scale, smem + OFF_Q + grp * BLK,
                      p.dk + head_off + (int64_t)kw0 * D, N - kw0, lane);
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

bool aligned_b(const void* ptr, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) % a) == 0;
}

template <int DT, int D, bool CAUSAL>
int launch_bwd_t(BwdParams prm, hipStream_t stream) {
  void* args[] = {&prm};
  prm.n_tiles = (prm.N + kDqT - 1) / kDqT;
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dq_kernel<DT, D, CAUSAL>),
                                 dim3((unsigned)(prm.bh * prm.n_tiles)), dim3(kDqThreads), args,
                                 0, stream);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  prm.n_tiles = (prm.N + kBT - 1) / kBT;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<DT, D, CAUSAL>),
                      dim3((unsigned)(prm.bh * prm.n_tiles)), dim3(kKVThreads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int DT>
int launch_bwd_dt(const BwdParams& prm, int d, int causal, hipStream_t s) {
  if (d == 64)
    return causal ? launch_bwd_t<DT, 64, true>(prm, s) : launch_bwd_t<DT, 64, false>(prm, s);
  return causal ? launch_bwd_t<DT, 128, true>(prm, s) : launch_bwd_t<DT, 128, false>(prm, s);
}

}  // namespace

extern "C" int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, float* dq, float* dk, float* dv, float* delta,
                      int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                      int dtype, void* stream) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_DTYPE_FP16 && dtype != FA_DTYPE_BF16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_CAUSAL;
  if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  // B and H are bounded one at a time first, so that B * H cannot overflow.
  if (N > (int64_t)1 << 22 || B > (int64_t)1 << 24 || H > (int64_t)1 << 24 ||
      B * H > (int64_t)1 << 24)
    return FA_ERR_SHAPE;
  if (B * H * ((N + kBT - 1) / kBT) > INT32_MAX) return FA_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
  if (!aligned_b(q, 16) || !aligned_b(k, 16) || !aligned_b(v, 16) || !aligned_b(o, 16) ||
      !aligned_b(dout, 16) || !aligned_b(dq, 16) || !aligned_b(dk, 16) || !aligned_b(dv, 16) ||
      !aligned_b(lse, 16) || !aligned_b(delta, 16))
    return FA_ERR_ALIGN;
  BwdParams prm;
  prm.q = static_cast<const uint8_t*>(q);
  prm.k = static_cast<const uint8_t*>(k);
  prm.v = static_cast<const uint8_t*>(v);
  prm.o = static_cast<const _Float16*>(o);
  prm.lse = lse;
  prm.dout = static_cast<const uint8_t*>(dout);
  prm.dq = dq;
  prm.dk = dk;
  prm.dv = dv;
  prm.delta = delta;
  prm.N = (int)N;
  prm.n_tiles = 0;
  prm.bh = (int)(B * H);
  prm.n_xcd = device_topology().xcds;
  prm.scale = scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == FA_DTYPE_BF16 ? launch_bwd_dt<FA_DTYPE_BF16>(prm, (int)d, causal, s)
                                : launch_bwd_dt<FA_DTYPE_FP16>(prm, (int)d, causal, s);
}
