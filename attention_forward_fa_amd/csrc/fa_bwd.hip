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
//   * fa_bwd_dq: one workgroup per (b, h, 128-query tile), a wave per 32
//     queries, shaped like the forward: S^T = K Q^T and dP^T = V dO^T with Q
//     and dO held in registers as B operands, dS^T in registers, then
//     dQ^T += K^T dS^T with K^T read transposed (ds_read_b64_tr_b16) from the
//     row-major K block in LDS.  It also computes D_i for its queries from O
//     and dO and stores it (delta), for the second kernel.
//   * fa_bwd_dkdv: one workgroup per (b, h, 128-key tile), two waves per 32
//     keys: a P wave holds the keys' K rows, computes S = Q K^T and P per
//     64-query block, dV^T += dO^T P, and passes P through LDS to the dS wave,
//     which holds the V rows, computes dP = dO V^T, dS = P (dP - D) and
//     dK^T += Q^T dS; dO^T / Q^T are read transposed from the row-major
//     dO / Q blocks.
// Blocks stream global -> LDS (buffer_load ... lds, XOR-swizzled 16-byte
// chunks), one barrier per block: the dQ kernel double-buffers K and V and
// unrolls its loop by two (running to an even block count, the extra block
// fully masked); the dK/dV kernel keeps three Q stages and two dO stages and
// unrolls by six, leaving after the last block.  Every stage index is thus a
// constant.  Rows past N read as zeros and are masked, as are causal pairs
// (key j > query i).  P and dS enter the second products
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

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = kWave * kBwdWaves;
constexpr int kRW = 32;                 // rows owned by one wave
constexpr int kBT = kRW * kBwdWaves;    // rows owned by one workgroup
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
template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void fa_bwd_dq_kernel(BwdParams p) {
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

  const int q0 = qt * kBT;
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
  BlockLoader<ROWB> ld;
  ld.init(wave, lane);

  int kv_end = N;
  if constexpr (CAUSAL) kv_end = min(N, q0 + kBT);
  const int nblk = (kv_end + kBS - 1) / kBS;

  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};

  ld.load(krs, k_lds0, 0, kv_end);
  ld.load(vrs, v_lds0, 0, kv_end);
  bwd_barrier();

  auto step = [&](int j, const uint8_t* kb, const uint8_t* vb, uint8_t* kn,
                  uint8_t* vn) __attribute__((always_inline)) {
    ld.load(krs, kn, (j + 1) * kBS, kv_end);  // next block, in flight during this one
    ld.load(vrs, vn, (j + 1) * kBS, kv_end);
    f32x16 st[2], dpt[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      st[t2] = f32x16{};
      dpt[t2] = f32x16{};
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        st[t2] = mfma16<DT>(row_operand<ROWB>(kb, ka, t2, ks), qreg[ks], st[t2]);
        dpt[t2] = mfma16<DT>(row_operand<ROWB>(vb, ka, t2, ks), doreg[ks], dpt[t2]);
      }
    mfma_read_pipeline<4 * NKS, 1, 2>();
    __builtin_amdgcn_sched_barrier(0);
    // dS^T = P^T (dP^T - D), P^T = exp2(cs s - lse log2 e); masked pairs give 0.
    uint32_t dsw[2][2][4];
    const int kb0 = j * kBS;
    float pt[2][16];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int i = 0; i < 16; ++i) pt[t2][i] = __builtin_amdgcn_exp2f(fmaf(st[t2][i], cs, -lse_l2));
    // Only a block reaching past N or past the wave's first query needs the
    // mask (one uniform branch; exp2 of a masked score is replaced, never used).
    if (kb0 + kBS > N || (CAUSAL && kb0 + kBS - 1 > qw0)) {
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb0 + t2 * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
          bool keep = key < N;
          if constexpr (CAUSAL) keep = keep && key <= my_q;
          pt[t2][i] = keep ? pt[t2][i] : 0.0f;
        }
    }
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int i = 0; i < 16; i += 2)
        dsw[t2][i / 8][(i % 8) / 2] = pack2<DT>(pt[t2][i] * (dpt[t2][i] - dsum),
                                                pt[t2][i + 1] * (dpt[t2][i + 1] - dsum));
    __builtin_amdgcn_sched_barrier(0);
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          const u32x4 b = {dsw[t2][s][0], dsw[t2][s][1], dsw[t2][s][2], dsw[t2][s][3]};
          acc[t] = mfma16<DT>(tr_operand<ROWB>(kb, ka, t, 2 * t2 + s), b, acc[t]);
        }
    mfma_read_pipeline<4 * NDT, 2, 2>();
    bwd_barrier();
  };
  for (int j = 0; j < nblk; j += 2) {
    step(j, k_lds0, v_lds0, k_lds1, v_lds1);
    step(j + 1, k_lds1, v_lds1, k_lds0, v_lds0);
  }

  // The loop's last barrier has drained every load and LDS access: the K and
  // V stages (one 32 x D fp32 block each) are free for the row-wise store.
  static_assert(kBwdWaves == 4 && BLK == kRW * D * 4, "one 32 x D fp32 block per stage");
  uint8_t* sbuf = wave == 0 ? k_lds0 : wave == 1 ? k_lds1 : wave == 2 ? v_lds0 : v_lds1;
  store_rows_f32<D>(acc, p.scale, sbuf, p.dq + head_off + (int64_t)qw0 * D, N - qw0, lane);
}

// ---------------------------------------------------------------------------
// dK and dV in one pass over the query blocks, by two kinds of wave per
// 32-key group: the P wave computes S = Q K^T, P and dV^T += dO^T P, and hands
// P (in the input type) to the group's dS wave through LDS; the dS wave
// computes dP = dO V^T, dS = P (dP - D) and dK^T += Q^T dS.  Four products per
// block, where a dV pass and a dK pass of their own would take five (S twice);
// each wave holds one key operand and one accumulator, so all eight fit two
// waves per SIMD, and the two kinds' VALU work lands in different halves of
// the block, beside the other kind's matrix instructions.
// ---------------------------------------------------------------------------
constexpr int kKVWaves = 2 * kBwdWaves;  // waves 0-3: P, 4-7: dS, of key group wave % 4
constexpr int kKVThreads = kWave * kKVWaves;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int DT, int D, bool CAUSAL>
__global__ __launch_bounds__(kKVThreads, 1) void fa_bwd_dkdv_kernel(BwdParams p) {
  constexpr int ROWB = D * 2;
  constexpr int NKS = D / 16;
  constexpr int NDT = D / 32;
  constexpr int BLK = kBS * ROWB;
  constexpr int PBLK = kRW * kBS * 2;  // one group's P block in the input type
  // The P waves run one query block ahead of the dS waves: in step j a P
  // wave computes P of block j + 1 (from Q_{j+1}) and dV of block j, its dS
  // wave dS and dK of block j (from P_j, dO_j, Q_j), while Q_{j+2} and
  // dO_{j+1} stream in -- three Q stages, two dO stages, one barrier a step.
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[3][BLK];
  __shared__ __attribute__((aligned(16))) uint8_t do_lds[2][BLK];
  // LSE (times log2 e) and D of a block's 64 queries.
  __shared__ __attribute__((aligned(16))) float lse_lds[2][kBS];
  __shared__ __attribute__((aligned(16))) float d_lds[2][kBS];
  // P of each key group, from its P wave to its dS wave: lane l's 16 dwords
  // as four 16-byte pieces at (c * 64 + l) * 16, c = 0 .. 3.
  __shared__ __attribute__((aligned(16))) uint8_t p_lds[2][kBwdWaves][PBLK];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 31, hh = lane >> 5;
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
  const int my_k = k0 + grp * kRW + lr;
  const float cs = p.scale * kLog2e;

  // This lane's key row of K (P wave) or V (dS wave): the B operand of
  // S = Q K^T or dP = dO V^T.
  u32x4 kv[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
    kv[ks] = __builtin_amdgcn_raw_buffer_load_b128(kvrs, my_k * ROWB + (ks * 16 + 8 * hh) * 2, 0, 0);

  BlockAddr<ROWB> qa;
  qa.init(lane);
  BlockLoader<ROWB, kKVWaves> ld;
  ld.init(wave, lane);

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
  // multiplied by log2 e, once per row instead of once per score.
  float lse_next = 0.0f;
  auto load_lse = [&](int row0) __attribute__((always_inline)) {
    const int off = (row0 < N ? row0 : N) * 4 + lane * 4;  // past N: zeros
    if (wave == 0) lse_next = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lrs, off, 0, 0));
  };
  auto store_lse = [&](float* lse_dst) __attribute__((always_inline)) {
    if (wave == 0) lse_dst[lane] = lse_next * kLog2e;
  };
  auto load_d = [&](float* d_dst, int row0) __attribute__((always_inline)) {
    const int off = (row0 < N ? row0 : N) * 4 + lane * 4;
    if (wave == 1) buffer_to_lds4(drs, d_dst, off);
  };

  // P of block j (P wave): S = Q K^T from Q block qb, exp2 against the
  // block's LSE, masked pairs 0, as pairs of the input type in w.  Elements
  // 4 g .. 4 g + 3 of tile t2 are query rows t2*32 + 8 g + 4 hh .. +3, whose
  // LSE log2 e (and D) are four consecutive floats; they go to k-step g / 2,
  // dwords 2 (g % 2), +1.  The P goes to LDS at px, for the dS wave and for
  // the P wave's own dV product a step later.
  auto p_block = [&](int j, const uint8_t* qb, const float* lb, uint8_t* px)
      __attribute__((always_inline)) {
    const int qrow0 = row0_of(j);
    uint32_t w[2][2][4];
    f32x16 x[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) x[t2] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
        x[t2] = mfma16<DT>(row_operand<ROWB>(qb, qa, t2, ks), kv[ks], x[t2]);
    mfma_read_pipeline<2 * NKS, 1, 4>();
    __builtin_amdgcn_sched_barrier(0);
    // Only a block reaching past N or below the tile's last key needs the
    // mask (a uniform branch; exp2 of a masked score is replaced, never used).
    const bool edge = qrow0 + kBS > N || (CAUSAL && qrow0 < k0 + kBT);
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lb + t2 * 32 + 8 * g + 4 * hh);
        float pt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pt[i] = __builtin_amdgcn_exp2f(fmaf(x[t2][4 * g + i], cs, -lse4[i]));
        if (edge) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int qi = qrow0 + t2 * 32 + 8 * g + 4 * hh + i;
            bool keep = qi < N;
            if constexpr (CAUSAL) keep = keep && qi >= my_k;
            pt[i] = keep ? pt[i] : 0.0f;
          }
        }
        w[t2][g / 2][2 * (g % 2)] = pack2<DT>(pt[0], pt[1]);
        w[t2][g / 2][2 * (g % 2) + 1] = pack2<DT>(pt[2], pt[3]);
      }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *reinterpret_cast<u32x4*>(px + (c * kWave + lane) * 16) =
          u32x4{w[c / 2][c % 2][0], w[c / 2][c % 2][1], w[c / 2][c % 2][2], w[c / 2][c % 2][3]};
  };

  // The 16 dwords of a P block that this lane wrote (or its partner wave's
  // lane wrote) at px.
  auto read_p = [&](const uint8_t* px, uint32_t (&w)[2][2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 pv = *reinterpret_cast<const u32x4*>(px + (c * kWave + lane) * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) w[c / 2][c % 2][e] = pv[e];
    }
  };

  // acc += (block tb)^T w: dV^T += dO^T P or dK^T += Q^T dS.
  auto second = [&](const uint8_t* tb, const uint32_t (&w)[2][2][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          const u32x4 b = {w[t2][sg][0], w[t2][sg][1], w[t2][sg][2], w[t2][sg][3]};
          acc[t] = mfma16<DT>(tr_operand<ROWB>(tb, qa, t, 2 * t2 + sg), b, acc[t]);
        }
    mfma_read_pipeline<4 * NDT, 2, 4>();
  };

  ld.load(qrs, q_lds[0], row0_of(0), N);
  ld.load(qrs, q_lds[1], row0_of(1), N);
  ld.load(dors, do_lds[0], row0_of(0), N);
  load_d(d_lds[0], row0_of(0));
  load_lse(row0_of(0));
  store_lse(lse_lds[0]);
  load_lse(row0_of(1));
  store_lse(lse_lds[1]);
  bwd_barrier();
  if (pw) p_block(0, q_lds[0], lse_lds[0], p_lds[0][grp]);
  bwd_barrier();

  // Step j; stage indices are j mod 3 (Q) and j mod 2 (the rest), fixed per
  // unrolled copy U = j mod 6.
  auto step = [&](int j, auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    constexpr int Q0 = U % 3, Q1 = (U + 1) % 3, Q2 = (U + 2) % 3, S0 = U % 2, S1 = (U + 1) % 2;
    ld.load(qrs, q_lds[Q2], row0_of(j + 2), N);
    ld.load(dors, do_lds[S1], row0_of(j + 1), N);
    load_d(d_lds[S1], row0_of(j + 1));
    load_lse(row0_of(j + 2));
    if (pw) {
      // dV^T += dO_j^T P_j, P_j read back from LDS; then P of block j + 1.
      uint32_t w[2][2][4];
      read_p(p_lds[S0][grp], w);
      second(do_lds[S0], w);
      __builtin_amdgcn_sched_barrier(0);
      if (j + 1 < nblk) p_block(j + 1, q_lds[Q1], lse_lds[S1], p_lds[S1][grp]);
    } else {
      // dP = dO V^T, then dS = P (dP - D) from the P wave's P, which is 0 at
      // every masked pair.
      f32x16 x[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) x[t2] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          x[t2] = mfma16<DT>(row_operand<ROWB>(do_lds[S0], qa, t2, ks), kv[ks], x[t2]);
      mfma_read_pipeline<2 * NKS, 1, 4>();
      __builtin_amdgcn_sched_barrier(0);
      uint32_t ds[2][2][4];
      read_p(p_lds[S0][grp], ds);
      const float* dlb = d_lds[S0];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(dlb + t2 * 32 + 8 * g + 4 * hh);
          float v4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            v4[i] = elem<DT>(ds[t2][g / 2][2 * (g % 2) + i / 2], i % 2) * (x[t2][4 * g + i] - d4[i]);
          ds[t2][g / 2][2 * (g % 2)] = pack2<DT>(v4[0], v4[1]);
          ds[t2][g / 2][2 * (g % 2) + 1] = pack2<DT>(v4[2], v4[3]);
        }
      __builtin_amdgcn_sched_barrier(0);
      second(q_lds[Q0], ds);
    }
    store_lse(lse_lds[S0]);  // LSE of block j + 2; lse_lds[S0] held block j's, used in step j - 1
    bwd_barrier();
  };
  for (int j = 0; j < nblk; j += 6) {
    step(j, std::integral_constant<int, 0>{});
    if (j + 1 >= nblk) break;
    step(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 >= nblk) break;
    step(j + 2, std::integral_constant<int, 2>{});
    if (j + 3 >= nblk) break;
    step(j + 3, std::integral_constant<int, 3>{});
    if (j + 4 >= nblk) break;
    step(j + 4, std::integral_constant<int, 4>{});
    if (j + 5 >= nblk) break;
    step(j + 5, std::integral_constant<int, 5>{});
  }

  // Every stage is free after the loop's last barrier: dV leaves through
  // four of them first, then dK.
  static_assert(kBwdWaves == 4 && BLK == kRW * D * 4, "one 32 x D fp32 block per stage");
  uint8_t* sbuf = grp < 3 ? q_lds[grp] : do_lds[0];
  const int kw0 = k0 + grp * kRW;
  if (pw) store_rows_f32<D>(acc, 1.0f, sbuf, p.dv + head_off + (int64_t)kw0 * D, N - kw0, lane);
  lds_barrier();
  if (!pw) store_rows_f32<D>(acc, p.scale, sbuf, p.dk + head_off + (int64_t)kw0 * D, N - kw0, lane);
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

bool aligned_b(const void* ptr, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) % a) == 0;
}

template <int DT, int D, bool CAUSAL>
int launch_bwd_t(BwdParams prm, hipStream_t stream) {
  prm.n_tiles = (prm.N + kBT - 1) / kBT;
  void* args[] = {&prm};
  const dim3 grid((unsigned)(prm.bh * prm.n_tiles));
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dq_kernel<DT, D, CAUSAL>),
                                 grid, dim3(kBwdThreads), args, 0, stream);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_bwd_dkdv_kernel<DT, D, CAUSAL>), grid,
                      dim3(kKVThreads), args, 0, stream);
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
