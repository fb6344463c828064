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
//   * each wave of 64 lanes owns 32 query rows; a workgroup of 8 waves
//     (fp16 / bf16, d = 128: one workgroup per CU, two waves per SIMD) or 4
//     waves (fp8: two workgroups per CU; d = 64: three) covers BR = 256 or
//     128 rows of one (b, h) head, and the whole K/V sequence streams past
//     it in blocks of BC = 64 keys (launch_t also picks 8 waves for d = 64
//     with long tiles, and for fp8 at d = 128 with P V in fp16 on grids of
//     two or more 256-row tiles per CU);
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_{f16,bf16} (or the fp8 v_mfma_scale_f32_32x32x64
//     with unit block scales), Q held in registers as the B operand.  In the
//     32x32 accumulator layout a lane owns one column (= one query) and 16
//     rows (= keys), so the row max / row sum of the softmax are in-lane
//     reductions plus one exchange with the lane 32 apart (v_permlane32_swap);
//   * the same accumulator registers, rounded to fp16, are already the B
//     operand of O^T += V^T P^T: the key order inside one MFMA's contraction
//     is free, so P never moves between lanes or through LDS;
//   * K goes global -> LDS directly (buffer_load ... lds) into rows whose
//     16-byte chunks carry an XOR swizzle, so the operand reads are free of
//     bank conflicts; V goes through registers, is converted to fp16 and
//     stored transposed (V^T rows, keys permuted inside groups of 16) so each
//     P V operand is one ds_read_b128;
//   * per-head buffer resources return zeros past row N, so ragged tails need
//     no bounds branches (keys past N are masked to -inf in the scores);
//   * software pipeline: iteration j issues the loads of K(j+3) and V(j+1)
//     and, in one run of MFMAs, P V of block j-1 followed by QK^T of block
//     j+1, with the softmax of block j and the V^T store of block j placed
//     between the MFMAs -- one matrix instruction per slice of the run, each
//     followed by a few vector instructions whose inputs are a slice old;
//     one workgroup barrier per block;
//   * the probabilities of a row are taken against a reference that starts
//     at the first block's max and moves only when a block's fp16
//     probabilities would approach the top of the fp16 range (a row-sum
//     check per block; the block is then redone against its own max), so no
//     per-block max reduction runs in the loop and O, l stay consistent
//     (fp8 P V keeps a per-block max: it sets the e4m3 scale);
//   * workgroups are mapped to XCDs by head so the query tiles of a head,
//     which all read the same K and V, share one L2.
// Further modes of the same kernel: a 4-wave twin of the 8-wave kernels for
// grids that would leave most CUs idle; fp8 P V (V kept as e4m3 in LDS and
// read with ds_read_b64_tr_b8, P rounded to e4m3 under a per-row power-of-two
// scale the MFMA takes back); and a key-range split, where long query tiles'
// key ranges are cut into chunks over several workgroups and fa_merge_kernel
// combines the chunks' O and LSE.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>
#include <stdint.h>
#include <type_traits>

#include "fa_common.h"
#include "fa_mi355x.h"

namespace {

constexpr int kQW = 32;            // query rows per wave
constexpr int kBC = 64;            // keys per K/V block
// The reference max of a row moves only when a block max passes it by more
// than this many powers of two, bounding every probability by 2^8 (fine for
// fp16 P) while skipping nearly all accumulator rescales.
constexpr float kRescaleLog2 = 8.0f;


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

// Waves per workgroup by default.  Eight (one workgroup per CU, two waves per
// SIMD) where a block carries 32 MFMAs per wave (fp16 / bf16 at d = 128);
// four (two workgroups per CU, three at d = 64, which drift apart and fill
// each other's barrier waits) where a block has fewer MFMAs per softmax
// instruction (d = 64, fp8).
// The eight-wave kernels have a four-wave twin (128-row tiles, one wave per
// SIMD) for grids that would leave most CUs idle; launch_t takes eight waves
// for some four-wave cases (d = 64 with long tiles, fp8 with P V in fp16),
// where staging K and V once for 256 rows pays.
template <int DT, int D>
constexpr int default_waves() { return (D == 128 && DT != FA_DTYPE_FP8_E4M3) ? 8 : 4; }
template <int WAVES>
struct Shape {
  static constexpr int waves = WAVES;
  static constexpr int threads = kWave * waves;
  static constexpr int br = kQW * waves;  // query rows per workgroup
};
constexpr int kMinBR = kQW * 4;           // smallest query tile of any kernel

// Workgroups a CU must hold at once (the register budget follows): two
// (two waves per SIMD), or three for the 4-wave d = 64 kernels, whose 50 KiB
// of LDS leave room for a third workgroup when the registers allow it.
template <int D, int WAVES>
constexpr int min_wgs_per_cu() { return (D == 64 && WAVES == 4) ? 3 : 2; }

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

// O^T += V^T P^T on the fp8 matrix cores: A = 32 e4m3 values of V^T per lane,
// B = 32 e4m3 probabilities per lane, each lane's B values multiplied by
// 2^(sb - 127) (an E8M0 exponent; one per lane, i.e. per query and half of the
// 64-key contraction).
__device__ __forceinline__ f32x16 mfma_pv8(const i32x8& a, const i32x8& b, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, sb);
}

// One run of NA MFMAs fed by RA LDS reads each, then NB MFMAs fed by RB
// reads each.  The reads run LA MFMAs ahead; after every MFMA come VPM VALU
// instructions and TPM transcendental ones (v_exp_f32 and the like form a
// class of their own for the scheduler); after MFMAs 3 .. 3+NW-1 one LDS
// write each, and after MFMAs
// VM0 .. VM0+NVM-1 one global load each, so the staging of the next block
// hides behind the matrix work too.
template <int NA, int RA, int NB, int RB, int LA, int VPM, int TPM, int NW, int NVM, int VM0 = 5,
          int I = 0>
__device__ __forceinline__ void mfma_run_pipeline() {
  constexpr int NM = NA + NB;
  static_assert(LA <= NM && VM0 + NVM <= NM, "run too short");
  if constexpr (I == 0)  // reads of the first LA MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, LA <= NA ? LA * RA : NA * RA + (LA - NA) * RB, 0);
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA I
    if constexpr (I + LA < NM)
      __builtin_amdgcn_sched_group_barrier(0x100, I + LA < NA ? RA : RB, 0);  // reads of I+LA
    if constexpr (I >= 3 && I < 3 + NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    if constexpr (I >= VM0 && I < VM0 + NVM) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // VALU
    __builtin_amdgcn_sched_group_barrier(0x400, TPM, 0);  // transcendental
    mfma_run_pipeline<NA, RA, NB, RB, LA, VPM, TPM, NW, NVM, VM0, I + 1>();
  }
}


// Two consecutive storage elements of V (one dword, fp16 or bf16) as fp16x2;
// or, for fp8, two e4m3 codes from the low / high 16 bits of a dword.
// fp8 codes are multiplied by the power of two pow2 (exact unless the result
// leaves the fp16 range).
template <int DT, bool HI_WORD>
__device__ __forceinline__ uint32_t v_pair_to_f16(uint32_t w, float pow2 = 1.0f) {
  if constexpr (DT == FA_DTYPE_FP16) {
    return w;
  } else if constexpr (DT == FA_DTYPE_BF16) {
    // bf16 -> fp32 is exact (upper half of a binary32); fp32 -> fp16 is exact for
    // every |v| in [2^-14, 65504] and rounds to nearest even below that.
    float lo = __uint_as_float(w << 16);
    float hi = __uint_as_float(w & 0xffff0000u);
    return pack_f16x2(lo, hi);
  } else {
    // The conversion's scale operand contributes its exponent only.
    f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, pow2, HI_WORD);  // exact
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
  int N;
  int H;
  int n_qtiles;  // query tiles of this launch (with the key-range split: of a head)
  int bh;      // B*H
  int layout;  // FA_LAYOUT_BHND or FA_LAYOUT_BNHD (q, k, v and o alike)
  int qt_base; // first query tile of this launch (n_qtiles tiles from there)
  int n_xcd;   // XCDs of the device (workgroup -> XCD mapping of tile_of)
  float scale;
  // Key-range split (split_g > 0): workgroup w takes head w % bh and the
  // (w / bh)-th chunk of that head, longest tiles first.  A tile's key range,
  // in groups of BR/64 blocks (causal tile t: t + 1 groups; otherwise
  // ceil(N / BR)), is cut into ceil(groups / split_g) chunks of near-equal
  // size.  Tiles with one chunk write O and LSE; the others write their
  // chunk's O (normalised, rounded to fp16) and LSE to ws_o / ws_lse, slot
  // ((bh * n_qtiles + t) * split_cmax + chunk) * BR + row, for the merge.
  int split_g;
  int split_cmax;
  _Float16* ws_o;
  float* ws_lse;
  // Per-key-tile fp8 scales (kernels with KVT): descale_k and descale_v hold
  // one scale per tile of kBC key rows, head bh's tile t at bh * n_kvt + t.
  int n_kvt;
};





// Swizzle of the fp8 V rows that the P V operand reads with
// ds_read_b64_tr_b8 (the 16-byte chunk XOR, from the row's place inside its
// group of 16 keys).  Those reads take, per half wave, the rows of one half
// of a 16-key group (keys 0-3 and 8-11, or 4-7 and 12-15) at the two chunks of
// 32 d values; with rows of 128 bytes an even and an odd row sit 64 banks
// apart, so the four rows of each parity need four distinct even XORs; with
// rows of 64 bytes rows r and r+8 meet and differ by an XOR of 2.
template <int ROWB>
__device__ __forceinline__ int vswz8(int row) {
  if constexpr (ROWB == 128) return (((row >> 1) & 1) << 1) | (((row >> 3) & 1) << 2);
  else return ((row >> 3) & 1) << 1;
}

// PV8: fp8 inputs with P V on the fp8 matrix cores too (V kept as e4m3 in
// LDS, P rounded to e4m3 under a per-row power-of-two scale); otherwise P V
// runs in fp16.  KVT: fp8 with K and V dequantization scales per key tile
// (one per block of kBC keys) instead of per head.
template <int DT, int D, bool CAUSAL, int WAVES, bool PV8 = false, bool KVT = false>
__global__ __launch_bounds__((Shape<WAVES>::threads), (min_wgs_per_cu<D, WAVES>()))
void fa_fwd_kernel(Params p) {
  using E = Elem<DT>;
  constexpr int kWaves = Shape<WAVES>::waves;
  constexpr int kThreads = Shape<WAVES>::threads;
  constexpr int kBR = Shape<WAVES>::br;
  constexpr int ES = E::bytes;
  constexpr int KROWB = D * ES;           // bytes per K row, global and LDS
  constexpr int KCPR = KROWB / 16;        // 16-byte chunks per K row
  constexpr int KBUF = kBC * KROWB;       // bytes of one K stage
  // V is stored transposed, V^T[d][key] in fp16, one row of kBC keys per d
  // value, padded by 16 bytes so that 16 consecutive rows read at one column
  // hit distinct banks.  Inside every group of 16 keys the two middle quads
  // are swapped (keys 0-3, 8-11, 4-7, 12-15), so the 8 keys one lane feeds to
  // a P V MFMA are contiguous.
  constexpr int VTROW = kBC * 2 + 16;     // bytes per V^T row
  constexpr int VBUF = D * VTROW;         // bytes of one V stage
  constexpr int NKS = D / E::kstep;       // QK^T MFMAs per 32x32 score tile
  constexpr int NDT = D / 32;             // 32-row d tiles of O^T
  constexpr int K_INSTR = kBC * KCPR / kWave;  // 64-lane LDS-load instructions per K stage
  constexpr int VD = kBC * D / (4 * kThreads);  // d values per staging thread (4 keys each)
  constexpr int VIN = VD * ES;            // input bytes per key row per staging thread
  static_assert(kBC * D == 4 * VD * kThreads, "V staging must tile the workgroup");
  static_assert(!PV8 || (DT == FA_DTYPE_FP8_E4M3 && WAVES == 4), "fp8 P V: fp8, four waves");
  static_assert(!KVT || DT == FA_DTYPE_FP8_E4M3, "per-tile scales: fp8 only");
  // fp16 P V: two V^T stages; fp8 P V: four stages of V rows as loaded.
  constexpr int VSTAGE = PV8 ? KBUF : VBUF;

  // Four K stages (K is loaded three blocks ahead of its use) and two V^T
  // stages, each an array of its own: the compiler can then tell the buffer
  // an LDS load is filling from the ones being read, and neither waits for
  // that load before the reads nor keeps the staging out of the MFMA run.
  __shared__ __attribute__((aligned(16))) uint8_t k_lds0[KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds1[KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds2[KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t k_lds3[KBUF];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds0[VSTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds1[VSTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds2[PV8 ? KBUF : 16];
  __shared__ __attribute__((aligned(16))) uint8_t v_lds3[PV8 ? KBUF : 16];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lr = lane & 31;   // row/column inside a 32x32 MFMA tile
  const int hh = lane >> 5;   // half of the wave

  // ---- work decomposition: one workgroup per (b*H + h, query tile) ----------
  int bh, qt;
  // Key blocks [kb_lo, kb_hi) of the tile's range; n_chunks > 1 when the
  // range is split over several workgroups.
  int kb_lo = 0, kb_hi = 0, chunk = 0, n_chunks = 1, n_groups = 0;
  if (p.split_g > 0) {
    bh = blockIdx.x % p.bh;
    int u = blockIdx.x / p.bh;
    const int g = p.split_g;
    if (CAUSAL) {
      qt = p.n_qtiles - 1;
      while (u >= (qt + g) / g) {  // tile qt: ceil((qt + 1) / g) chunks
        u -= (qt + g) / g;
        --qt;
      }
      n_groups = qt + 1;
    } else {
      n_groups = (p.N + kBR - 1) / kBR;
      const int per_tile = (n_groups + g - 1) / g;
      qt = u / per_tile;
      u -= qt * per_tile;
    }
    chunk = u;
    n_chunks = (n_groups + g - 1) / g;
  } else {
    tile_of(blockIdx.x, p.bh, p.n_qtiles, CAUSAL, p.n_xcd, bh, qt);
    qt += p.qt_base;
  }
  const int N = p.N;
  // Element offset of the head's first row and the stride between its rows:
  // [B, H, N, d] (rows of one head adjacent) or [B, N, H, d] (rows of one head
  // H*d elements apart).  Q, K, V and O share the layout.
  int64_t head_off;
  int row_elems;
  if (p.layout == FA_LAYOUT_BNHD) {
    const int b = bh / p.H, h = bh - b * p.H;
    head_off = ((int64_t)b * N * p.H + h) * D;
    row_elems = p.H * D;
  } else {
    head_off = (int64_t)bh * N * D;
    row_elems = D;
  }
  const int GRS = row_elems * ES;             // bytes between rows in global memory
  const int head_bytes = (N - 1) * GRS + KROWB;  // <= 2^30, checked on the host
  const __amdgpu_buffer_rsrc_t qrs = head_rsrc(p.q + head_off * ES, head_bytes);
  const __amdgpu_buffer_rsrc_t krs = head_rsrc(p.k + head_off * ES, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = head_rsrc(p.v + head_off * ES, head_bytes);

  const int q0 = qt * kBR;              // first query row of the workgroup
  const int qw0 = q0 + wave * kQW;      // first query row of this wave
  const int my_q = qw0 + lr;            // the query held by this lane's column

  float c = p.scale * kLog2e;           // exp(x) = exp2(x log2 e)
  float v_scale = 1.0f;
  if constexpr (DT == FA_DTYPE_FP8_E4M3) {
    if (p.descale_q) {
      c *= p.descale_q[bh];
      if constexpr (!KVT) {
        c *= p.descale_k[bh];
        v_scale = p.descale_v[bh];
      }
    }
  }
  // Per-key-tile scales of block j (KVT).  K's scale multiplies the block's
  // scores: cb = c * descale_k.  V's scale dv = 2^ev * f, f in [1, 2), is
  // split: 2^ev is applied exactly where V's e4m3 values are converted to
  // fp16 (or, for fp8 P V, in the matrix instruction's E8M0 scale of P) and f
  // multiplies the block's probabilities inside their exponential (log2 f
  // added to the exponent), the row sum dividing it out again.  Scales must
  // be positive normal floats.
  struct TileScale {
    float cb = 0.0f, lf = 0.0f, inv_f = 1.0f, vp2 = 1.0f;
    int ev = 0;
  };
  // The raw K and V scales of a block are loaded one block ahead, by vector
  // loads of a uniform address: a scalar load in flight would make every LDS
  // wait of the loop wait for it too (the two share one counter and return
  // out of order).  Issued before the block's K and V loads, so the wait for
  // those at the end of an iteration covers them.
  float sk_next = 0.0f, sv_next = 0.0f;
  const __amdgpu_buffer_rsrc_t dks = head_rsrc(
      reinterpret_cast<const uint8_t*>(p.descale_k + (KVT ? (int64_t)bh * p.n_kvt : 0)),
      KVT ? p.n_kvt * 4 : 0);
  const __amdgpu_buffer_rsrc_t dvs = head_rsrc(
      reinterpret_cast<const uint8_t*>(p.descale_v + (KVT ? (int64_t)bh * p.n_kvt : 0)),
      KVT ? p.n_kvt * 4 : 0);
  auto load_scales = [&](int j) __attribute__((always_inline)) {
    if constexpr (KVT) {
      const int off = min(j, p.n_kvt - 1) * 4;  // blocks past N: any tile's
      sk_next = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dks, off, 0, 0));
      sv_next = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dvs, off, 0, 0));
    }
  };
  auto tile_scale = [&](float sk, float sv) __attribute__((always_inline)) {
    TileScale t;
    if constexpr (KVT) {
      const uint32_t vb = __float_as_uint(sv);
      t.cb = c * sk;
      t.vp2 = __uint_as_float(vb & 0xff800000u);                 // 2^ev
      const float f = __uint_as_float((vb & 0x007fffffu) | 0x3f800000u);  // [1, 2)
      t.lf = __builtin_amdgcn_logf(f);
      t.inv_f = __builtin_amdgcn_rcpf(f);
      t.ev = (int)((vb >> 23) & 0xffu) - 127;
    } else {
      t.cb = c;
    }
    return t;
  };

  // ---- Q tile -> registers, the B operand of S^T = K Q^T (rows >= N read 0) --
  QKOperand<DT> qreg[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    const int byte = (ks * E::kstep + hh * (E::kstep / 2)) * ES;
#pragma unroll
    for (int w = 0; w < E::opnd_dwords; w += 4) {
      u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(qrs, my_q * GRS + byte + 4 * w, 0, 0);
      qreg[ks].w[w + 0] = x[0];
      qreg[ks].w[w + 1] = x[1];
      qreg[ks].w[w + 2] = x[2];
      qreg[ks].w[w + 3] = x[3];
    }
  }

  // ---- K/V blocks this workgroup visits --------------------------------------
  int kv_end = N;
  if constexpr (CAUSAL) kv_end = min(N, q0 + kBR);
  kb_hi = (kv_end + kBC - 1) / kBC;
  if (n_chunks > 1) {
    // Chunk boundaries fall on whole groups, so the first block of a chunk
    // starts at or before the tile's first row (causal) and below N: every
    // row of the tile has a key in it, as the running max requires.
    constexpr int A = kBR / kBC;  // blocks per group
    kb_lo = A * (chunk * n_groups / n_chunks);
    kb_hi = min(kb_hi, A * ((chunk + 1) * n_groups / n_chunks));
    kv_end = min(kv_end, kb_hi * kBC);
  }

  // ---- staging -----------------------------------------------------------------
  // All eight waves stage.  K goes global -> LDS directly (buffer_load ...
  // lds): one instruction fills 64 consecutive 16-byte LDS slots, lane t slot
  // t; slot s of a stage holds row s / KCPR, physical chunk s % KCPR, so each
  // lane fetches the logical chunk the swizzle puts there.  V goes through
  // registers: thread (quad, dgrp) loads keys 4*quad .. +3 at d values
  // dgrp*VD .. +VD-1, converts them to fp16 and writes VD rows of V^T, 4 keys
  // (8 bytes) each, one iteration later.  Block offsets go into the VGPR
  // offset, which the buffer range check covers: rows at or past N read 0.
  // Blocks past the last one this workgroup needs are pointed beyond every
  // head's range, so they read 0 without touching memory.
  static_assert(K_INSTR % kWaves == 0, "K stage must split evenly over the waves");
  constexpr int K_PER_W = K_INSTR / kWaves;
  int k_goff[K_PER_W];
#pragma unroll
  for (int u = 0; u < K_PER_W; ++u) {
    const int slot = (u * kWaves + wave) * kWave + lane;
    const int row = slot / KCPR, phys = slot % KCPR;
    k_goff[u] = row * GRS + ((phys ^ swz<KROWB>(row)) * 16);
  }
  // fp8 P V: V rows go global -> LDS the same way, under their own swizzle.
  int v8_goff[K_PER_W];
#pragma unroll
  for (int u = 0; u < K_PER_W; ++u) {
    const int slot = (u * kWaves + wave) * kWave + lane;
    const int row = slot / KCPR, phys = slot % KCPR;
    v8_goff[u] = row * GRS + ((phys ^ vswz8<KROWB>(row)) * 16);
  }
  const int vquad = tid % 16, vdgrp = tid / 16;
  const int v_goff = 4 * vquad * GRS + vdgrp * VIN;
  int v_loff;
  {
    const int qq = vquad % 4;  // quad inside its 16-key group -> position quad
    const int keypos = 16 * (vquad / 4) + 4 * ((qq >> 1) + 2 * (qq & 1));
    v_loff = vdgrp * VD * VTROW + keypos * 2;
  }
  constexpr int VW = (VIN + 3) / 4;  // dwords of one key row of a staging thread
  typedef uint32_t VRegs[4][VW];     // one block's share of V, as loaded
  VRegs vst;
  // Byte offset of key row kb, or one past every valid offset (a head spans
  // at most 2^30 bytes) for a block the workgroup does not use.
  auto block_off = [&](int kb) __attribute__((always_inline)) { return kb < kv_end ? kb * GRS : (1 << 30); };

  auto load_k = [&](int kb, uint8_t* kbuf) __attribute__((always_inline)) {
    const int boff = block_off(kb);
#pragma unroll
    for (int u = 0; u < K_PER_W; ++u) {
      const int inst = u * kWaves + wave;
      buffer_to_lds16(krs, kbuf + inst * kWave * 16, k_goff[u] + boff, 0);
    }
  };
  auto load_v8 = [&](int kb, uint8_t* vbuf) __attribute__((always_inline)) {
    const int boff = block_off(kb);
#pragma unroll
    for (int u = 0; u < K_PER_W; ++u) {
      const int inst = u * kWaves + wave;
      buffer_to_lds16(vrs, vbuf + inst * kWave * 16, v8_goff[u] + boff, 0);
    }
  };
  auto load_v = [&](int kb, VRegs& vst) __attribute__((always_inline)) {
    const int boff = block_off(kb);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int off = v_goff + r * GRS + boff;
      if constexpr (VIN == 16) {
        u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, 0);
        vst[r][0] = x[0]; vst[r][1] = x[1]; vst[r][2] = x[2]; vst[r][3] = x[3];
      } else if constexpr (VIN == 8) {
        u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, 0);
        vst[r][0] = x[0]; vst[r][1] = x[1];
      } else if constexpr (VIN == 4) {
        vst[r][0] = __builtin_amdgcn_raw_buffer_load_b32(vrs, off, 0, 0);
      } else {
        vst[r][0] = __builtin_amdgcn_raw_buffer_load_b16(vrs, off, 0, 0);
      }
    }
  };
  // Convert the 4 x VD block held in registers to fp16 and write its VD rows
  // of V^T into the V^T buffer vbuf.
  auto store_v = [&](const VRegs& vst, uint8_t* vbuf, float vp2) __attribute__((always_inline)) {
    uint32_t h[4][VD / 2];  // fp16 pairs along d, per key
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int w = 0; w < VD / 2; ++w) {
        if constexpr (ES == 2) {
          h[r][w] = v_pair_to_f16<DT, false>(vst[r][w]);
        } else if (w & 1) {
          h[r][w] = v_pair_to_f16<DT, true>(vst[r][w / 2], vp2);
        } else {
          h[r][w] = v_pair_to_f16<DT, false>(vst[r][w / 2], vp2);
        }
      }
    // v_perm_b32 picks bytes of {a, b} (b = bytes 0-3, a = bytes 4-7): the
    // low halves of two keys for an even d, the high halves for an odd one.
#pragma unroll
    for (int e = 0; e < VD; ++e) {
      const int w = e / 2;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t lo = __builtin_amdgcn_perm(h[1][w], h[0][w], sel);
      const uint32_t hi = __builtin_amdgcn_perm(h[3][w], h[2][w], sel);
      *reinterpret_cast<u32x2*>(vbuf + v_loff + e * VTROW) = u32x2{lo, hi};
    }
  };
  // Workgroup barrier that leaves global loads in flight: this wave's LDS
  // accesses complete, then s_barrier.  (__syncthreads would also wait for
  // every outstanding global load.)  Loads that must have landed before it
  // are waited for explicitly with vmcnt.
  auto barrier = []() __attribute__((always_inline)) { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  // ---- per-lane LDS operand addresses (block-independent parts) -------------
  // K (A operand of S^T): row kt*32 + lr, logical chunk(s) of k-step ks.
  constexpr int KCH = E::opnd_dwords / 4;  // 16-byte chunks per operand
  int k_raddr[NKS][KCH];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int lc = (ks * E::kstep + hh * (E::kstep / 2)) * ES / 16 + u;
      k_raddr[ks][u] = lr * KROWB + ((lc ^ swz<KROWB>(lr)) * 16);
    }
  // V^T (A operand of O^T = V^T P^T): row t*32 + lr, the 8 contiguous key
  // positions 16*s + 8*hh .. +7 of key tile kt.
  const int vt_raddr = lr * VTROW + 16 * hh;
  // fp8 P V: the A operand (32 e4m3 values of V^T per lane) comes from the
  // row-major V block through four ds_read_b64_tr_b8.  In each group of 16
  // lanes, lane 2e+h gives the address of 8 bytes (columns 8h .. 8h+7 of a
  // 16-byte span) of row e of an 8 x 16-byte tile and lane L receives column L
  // of the tile's 8 rows.  Group g reads d columns t*32 + 16*(g&1) .. +15, and
  // in read r the rows are the keys behind bytes 8r .. 8r+7 of the B operand
  // of half g>>1: key 16r + 8*(e>>2) + 4*(g>>1) + (e&3).
  int vt8_addr[NDT];
  {
    const int g = lane >> 4, li = lane & 15, e = li >> 1;
    const int b = 8 * (e >> 2) + 4 * (g >> 1) + (e & 3);  // row inside its 16-key group
#pragma unroll
    for (int t = 0; t < NDT; ++t)
      vt8_addr[t] = b * KROWB + (((2 * t + (g & 1)) ^ vswz8<KROWB>(b)) * 16) + 8 * (li & 1);
  }

  // ---- running softmax state and the O^T accumulator --------------------------
  f32x16 acc[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) acc[t] = f32x16{};
  // Reference of this query's probabilities, p = exp2(c s - ref), in log2
  // units.  fp16 P V: ref_c, set from the first block's max and moved only
  // when a block's fp16 probabilities would come near the top of the fp16
  // range (the optimistic softmax below).  fp8 P V: ref8, moved when a block
  // max exceeds it by more than kRescaleLog2 (so p <= 2^kRescaleLog2).
  float ref_c = 0.0f;
  float ref8 = -INFINITY;
  float l_run = 0.0f;  // this lane's share of the row sum, relative to the reference
  // P as fp16 pairs, the B operand of O^T += V^T P^T: [key tile][k-step][dword].
  typedef uint32_t PRegs[2][2][4];
  // fp8 P V: P as 32 e4m3 codes (byte 16*kt + i = accumulator element i of key
  // tile kt), then the E8M0 exponent of the scale 2^-k they were taken under.
  typedef uint32_t P8Regs[9];

  // S^T = K Q^T for the block in K buffer kbuf: two 32-key tiles.  The tiles
  // alternate so consecutive MFMAs are independent.
  auto qk = [&](const uint8_t* kbuf, f32x16* st) __attribute__((always_inline)) {
    st[0] = f32x16{};
    st[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        QKOperand<DT> a;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
          u32x4 x = *reinterpret_cast<const u32x4*>(kbuf + kt * 32 * KROWB + k_raddr[ks][u]);
          a.w[4 * u + 0] = x[0]; a.w[4 * u + 1] = x[1];
          a.w[4 * u + 2] = x[2]; a.w[4 * u + 3] = x[3];
        }
        st[kt] = mfma_qk<DT>(a, qreg[ks], st[kt]);
      }
  };

  // Keys past N, and (causal) keys after the query, get score -inf.  A block
  // with every key masked for this lane leaves the reference and l_run unchanged and
  // contributes P = 0 (block 0 always holds a valid key for every row).
  auto needs_mask = [&](int j) __attribute__((always_inline)) {
    return (j * kBC + kBC > kv_end) || (CAUSAL && j * kBC + kBC - 1 > qw0);
  };
  auto mask = [&](f32x16* st, int kb) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb + kt * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
        bool keep = key < kv_end;
        if constexpr (CAUSAL) keep = keep && key <= my_q;
        st[kt][i] = keep ? st[kt][i] : -INFINITY;
      }
  };

  // Online softmax of one block against the current reference (fp16 P V), the
  // optimistic form: no block max is taken.  p = exp2(c s - ref_c) rounded to
  // fp16 pairs laid out as the B operand of O^T += V^T P^T, and the lane's
  // share of the block's row sum over those fp16 values.  Any reference keeps
  // O and l consistent (both scale alike), so ref_c only has to keep every p
  // finite and well inside the fp16 range: while the lane's share stays below
  // 2^15, every p does.  Returns that share; a lane at or above it (or NaN /
  // inf) sends the wave through rescale_block below.  The row's true max
  // enters only through the first block (ref_c starts at its max) and those
  // rare rescales, so the per-block chain max -> lane exchange -> exp of the
  // usual online softmax, and its VALU work, drop out of the loop.
  constexpr float kRowSumCap = 32768.0f;
  auto softmax = [&](f32x16* st, PRegs& pw, const TileScale& ts) __attribute__((always_inline)) -> float {
    const float nref = ts.lf - ref_c;
    // p = exp2(c s - ref) (times f, KVT): all FMAs, then all exponentials, in place.
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = fmaf(st[kt][i], ts.cb, nref);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = __builtin_amdgcn_exp2f(st[kt][i]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; i += 2) pw[kt][i / 8][(i % 8) / 2] = pack_f16x2(st[kt][i], st[kt][i + 1]);
    // Row sum of the fp16 probabilities that multiply V (so numerator and
    // denominator see the same rounding), two at a time with v_dot2_f32_f16
    // against (1, 1) in four independent chains.
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          part[w] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pw[kt][s][w]), ones, part[w],
                                           false);
    return (part[0] + part[1]) + (part[2] + part[3]);
  };

  // Raw scores' max over the block for this query (both lanes of the pair).
  auto block_max = [&](const f32x16* st) __attribute__((always_inline)) -> float {
    float m0 = st[0][0], m1 = st[1][0];  // two independent chains
#pragma unroll
    for (int i = 1; i < 15; i += 2) {
      m0 = vmax(vmax(m0, st[0][i]), st[0][i + 1]);
      m1 = vmax(vmax(m1, st[1][i]), st[1][i + 1]);
    }
    return max_pair32(vmax(vmax(m0, st[0][15]), vmax(m1, st[1][15])));
  };

  // O^T += V^T P^T for the block in V buffer vbuf.  Slot i of lane half hh
  // in k-step s of key tile kt is key kt*32 + 16*s + 8*(i/4) + 4*hh + (i%4),
  // the order the S^T accumulator holds and the order of V^T's permuted key
  // positions 16*s + 8*hh + i.  d tiles innermost: consecutive MFMAs update
  // different accumulators.
  auto pv = [&](const uint8_t* vbuf, const PRegs& pw) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int t = 0; t < NDT; ++t) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(
              vbuf + vt_raddr + t * 32 * VTROW + (kt * 32 + 16 * s) * 2);
          u32x4 b = {pw[kt][s][0], pw[kt][s][1], pw[kt][s][2], pw[kt][s][3]};
          acc[t] = mfma_pv(a, b, acc[t]);
        }
  };

  // fp8 P V softmax, in log2 units like the reference ref8: the row's block
  // max (scaled) moves the reference when it passes it by more than
  // kRescaleLog2; the probabilities are taken as 2^k exp2(cb s - ref8) (times
  // f, KVT) with k = 8 - ceil(block max - ref8 (+ log2 f)), which lifts the
  // block's largest one into (2^7, 2^8] (e4m3 holds 3 fraction bits from 2^-6
  // to 448), rounded to e4m3, and the MFMA scales them back by 2^-k (and 2^ev,
  // KVT).  The row sum takes the unrounded values.
  auto softmax8 = [&](f32x16* st, P8Regs& pw, bool& rescale, const TileScale& ts)
                      __attribute__((always_inline)) -> float {
    float m0 = st[0][0], m1 = st[1][0];
#pragma unroll
    for (int i = 1; i < 15; i += 2) {
      m0 = vmax(vmax(m0, st[0][i]), st[0][i + 1]);
      m1 = vmax(vmax(m1, st[1][i]), st[1][i + 1]);
    }
    const float mxs = max_pair32(vmax(vmax(m0, st[0][15]), vmax(m1, st[1][15]))) * ts.cb;
    rescale = __builtin_amdgcn_ballot_w64(mxs - ref8 > kRescaleLog2) != 0;
    const float ref_use = rescale ? vmax(ref8, mxs) : ref8;
    const float alpha = __builtin_amdgcn_exp2f(ref8 - ref_use);
    ref8 = ref_use;
    // mxs - ref_use <= kRescaleLog2 = 8 and log2 f < 1, so k >= -1 (2^-1 is an
    // exact E8M0 factor too); a row with no key in the block (mxs = -inf)
    // takes k = 64.
    const float kf = fminf(8.0f - ceilf(mxs - ref_use + ts.lf), 64.0f);
    const int ki = (int)kf;
    const float bias = kf + ts.lf - ref_use;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = fmaf(st[kt][i], ts.cb, bias);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) st[kt][i] = __builtin_amdgcn_exp2f(st[kt][i]);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int kt = w / 4, g = w % 4;
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(st[kt][4 * g], st[kt][4 * g + 1], 0, false);
      pw[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(st[kt][4 * g + 2], st[kt][4 * g + 3], lo,
                                                        true);
    }
    pw[8] = (uint32_t)(127 - ki + ts.ev);
    float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) part[i % 4] += st[kt][i];
    const float ls = __builtin_amdgcn_ldexpf((part[0] + part[1]) + (part[2] + part[3]), -ki);
    l_run = l_run * alpha + (KVT ? ls * ts.inv_f : ls);
    return alpha;
  };

  // fp8 P V: one MFMA per d tile covers the whole 64-key block; byte j of a
  // lane's B operand is key 32*(j/16) + 8*((j%16)/4) + 4*hh + (j%4), the key
  // the tr_b8 reads put in byte j of the A operand.
  auto pv8 = [&](const uint8_t* vbuf, const P8Regs& pw) __attribute__((always_inline)) {
    i32x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (int)pw[i];
    const int sb = (int)pw[8];
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      i32x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (lds_i32x2_t*)(vbuf + vt8_addr[t] + r * 16 * KROWB));
        a[2 * r] = x[0];
        a[2 * r + 1] = x[1];
      }
      acc[t] = mfma_pv8(a, b, sb, acc[t]);
    }
  };

  // ---- software pipeline ---------------------------------------------------------
  // Iteration j writes V(j) -- loaded into registers during iteration j-1 --
  // to V^T buffer j&1 (last read in iteration j-1), loads V(j+1) into the
  // freed registers and K(j+3) into K stage (j+3)%4 (which held K(j-1), read
  // in iteration j-2).  One run of MFMAs, P V of block j-1 (V^T buffer
  // (j-1)&1, P(j-1) kept from the previous iteration) followed by QK^T of
  // block j+1 (K stage (j+1)%4), carries the softmax of block j and the
  // staging in the issue slots between the MFMAs.  Each wave then waits for
  // its loads of the previous iteration (K(j+2) is read next iteration) --
  // those of this iteration stay in flight; V(j+1) is waited for where it is
  // stored -- and the workgroup meets at one barrier.  The loop is unrolled by four so every buffer is a
  // compile-time choice.  Loads are issued unconditionally (blocks past the
  // end read 0), so the loop body is a straight line and the outstanding-load
  // counts are fixed; the QK^T of the block after the last is computed and
  // discarded, and iteration 0 multiplies a zero P(-1) with the zeroed V^T
  // buffer 1.
  if constexpr (!PV8) {
    for (int i = tid; i < VBUF / 16; i += kThreads) {
      reinterpret_cast<u32x4*>(v_lds0)[i] = u32x4{0u, 0u, 0u, 0u};
      reinterpret_cast<u32x4*>(v_lds1)[i] = u32x4{0u, 0u, 0u, 0u};
    }
    constexpr int NVM = K_PER_W + 4;  // global load instructions per wave per iteration
    load_scales(kb_lo);
    load_k(kb_lo * kBC, k_lds0);
    load_k((kb_lo + 1) * kBC, k_lds1);
    load_v(kb_lo * kBC, vst);
    load_k((kb_lo + 2) * kBC, k_lds2);
    // This wave's K(0) and K(1) have landed; V(0) and K(2) may still fly.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 + K_PER_W) : "memory");
    barrier();

    f32x16 sa[2], sb[2];
    PRegs pa, pb = {};
    qk(k_lds0, sa);
    // The reference starts at the first block's max (every row has a key in
    // the first block of its range, so it is finite).
    if (needs_mask(kb_lo)) mask(sa, kb_lo * kBC);
    ref_c = block_max(sa) * tile_scale(sk_next, sv_next).cb;
    barrier();

    constexpr int NPV = NDT * 4;     // P V MFMAs per block
    constexpr int NQK = 2 * NKS;     // QK^T MFMAs per block
    // A block whose probabilities came too close to the top of the fp16 range
    // against the current reference (rare: the first block sets it, and the
    // fp16 range leaves 15 powers of two above it): S(j) again from K(j),
    // which stays in its LDS stage until the next iteration's loads; the
    // reference moves up to the block's max, O^T (which holds blocks up to
    // j - 1 once this iteration's P V has run) and l scale by
    // exp2(old - new), and P(j) is taken again.
    auto rescale_block = [&](int j, const uint8_t* k_cur, f32x16* st, PRegs& p_cur,
                             const TileScale& ts) __attribute__((always_inline)) -> float {
      qk(k_cur, st);  // into the registers of the block's spent fp32 probabilities
      mfma_read_pipeline<NQK, KCH, 1>();  // one operand read ahead: few registers in flight
      if (needs_mask(j)) mask(st, j * kBC);
      const float ref_new = vmax(ref_c, block_max(st) * ts.cb);  // a fully masked row keeps ref_c
      const float alpha = __builtin_amdgcn_exp2f(ref_c - ref_new);
      ref_c = ref_new;
      const float ls = softmax(st, p_cur, ts);
      l_run = l_run * alpha + (KVT ? ls * ts.inv_f : ls);
      return alpha;
    };
    // One iteration as an explicit software pipeline of NM slices.  Slice m
    // issues matrix instruction m of the run (P V of block j-1, then QK^T of
    // block j+1), the LDS operand reads of instruction m + LA, and slice m's
    // share of block j's softmax: score i's FMA in slice ~i*NM/32 - 1, its
    // exponential one slice later, the fp16 pack of a pair and its row-sum dot
    // product one and two slices after that.  A scheduling barrier closes
    // every slice, so each wave's stream alternates one matrix instruction
    // with a few independent vector instructions whose inputs were produced
    // at least a slice earlier -- the mix two waves of a SIMD overlap best
    // (matrix pipe busy while the other wave's vector work issues) -- instead
    // of runs of dependent vector work between runs of matrix instructions.
    constexpr int NM = NPV + NQK;
    constexpr int LA = 4;                          // operand reads issued ahead
    constexpr int OW = KCH * 4;                    // dwords of one operand
    static_assert(NM >= 8, "run too short for the slice schedule");
    auto fma_slice = [](int i) { return (i * NM) / 32 - 1; };  // slices -1 .. NM-1
    auto step = [&](int j, const uint8_t* k_cur, const uint8_t* k_next, uint8_t* k_fill,
                    const uint8_t* v_prev, uint8_t* v_fill, f32x16* s_cur, f32x16* s_next,
                    PRegs& p_cur, const PRegs& p_prev) __attribute__((always_inline)) {
      if (needs_mask(j)) mask(s_cur, j * kBC);
      const float sk = sk_next, sv = sv_next;
      load_scales(j + 1);
      const TileScale ts = tile_scale(sk, sv);
      uint32_t opnd[LA][OW];                       // operand ring, slot m % LA
      auto read = [&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m < NPV) {
          constexpr int kt = m / (2 * NDT), sidx = (m / NDT) % 2, t = m % NDT;
          const u32x4 x = *reinterpret_cast<const u32x4*>(
              v_prev + vt_raddr + t * 32 * VTROW + (kt * 32 + 16 * sidx) * 2);
#pragma unroll
          for (int w = 0; w < 4; ++w) opnd[m % LA][w] = x[w];
        } else {
          constexpr int q = m - NPV, ks = q / 2, kt = q % 2;
#pragma unroll
          for (int u = 0; u < KCH; ++u) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(k_next + kt * 32 * KROWB + k_raddr[ks][u]);
#pragma unroll
            for (int w = 0; w < 4; ++w) opnd[m % LA][4 * u + w] = x[w];
          }
        }
      };
      auto mfma = [&](auto mc) __attribute__((always_inline)) {
        constexpr int m = decltype(mc)::value;
        if constexpr (m < NPV) {
          constexpr int kt = m / (2 * NDT), sidx = (m / NDT) % 2, t = m % NDT;
          const u32x4 a = {opnd[m % LA][0], opnd[m % LA][1], opnd[m % LA][2], opnd[m % LA][3]};
          const u32x4 b = {p_prev[kt][sidx][0], p_prev[kt][sidx][1], p_prev[kt][sidx][2],
                           p_prev[kt][sidx][3]};
          acc[t] = mfma_pv(a, b, acc[t]);
        } else {
          constexpr int q = m - NPV, ks = q / 2, kt = q % 2;
          QKOperand<DT> a;
#pragma unroll
          for (int w = 0; w < OW; ++w) a.w[w] = opnd[m % LA][w];
          s_next[kt] = mfma_qk<DT>(a, qreg[ks], ks == 0 ? f32x16{} : s_next[kt]);
        }
      };
      const float nref = ts.lf - ref_c;
      float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
      auto softmax_slice = [&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          if (fma_slice(i) == k) s_cur[i / 16][i % 16] = fmaf(s_cur[i / 16][i % 16], ts.cb, nref);
          if (fma_slice(i) + 1 == k) s_cur[i / 16][i % 16] = __builtin_amdgcn_exp2f(s_cur[i / 16][i % 16]);
          if (i % 2 == 1 && fma_slice(i) + 2 == k) {
            const int kt = i / 16, e = i % 16 - 1;
            p_cur[kt][e / 8][(e % 8) / 2] = pack_f16x2(s_cur[kt][e], s_cur[kt][e + 1]);
          }
          if (i % 2 == 1 && fma_slice(i) + 3 == k) {
            const int kt = i / 16, e = i % 16 - 1, pi = i / 2;
            part[pi % 4] = __builtin_amdgcn_fdot2(
                __builtin_bit_cast(f16x2, p_cur[kt][e / 8][(e % 8) / 2]), ones, part[pi % 4], false);
          }
        }
      };
      // slice -1: the first LA operand reads and the first scores' FMAs
      static_for<0, LA>(read);
      softmax_slice(std::integral_constant<int, -1>{});
      __builtin_amdgcn_sched_barrier(0);
      static_for<0, NM + 3>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < NM) mfma(kc);
        if constexpr (k + LA < NM) read(std::integral_constant<int, k + LA>{});
        softmax_slice(kc);
        if constexpr (k == 0) store_v(vst, v_fill, ts.vp2);    // V(j) -> V^T
        if constexpr (k == 2) load_v((j + 1) * kBC, vst);      // V(j+1) -> registers
        if constexpr (k == 4) load_k((j + 3) * kBC, k_fill);   // K(j+3), after V(j+1)
        __builtin_amdgcn_sched_barrier(0);
      });
      const float ls = (part[0] + part[1]) + (part[2] + part[3]);
      const bool big = __builtin_amdgcn_ballot_w64(!(ls < kRowSumCap)) != 0;
      float alpha = 1.0f;
      if (big) {
        // The recomputed P is moved into the registers of the block's first P
        // by moves whose result is tied to their destination (DPP with the
        // identity pattern).  Left to itself the register allocator gave the
        // two paths' P different homes and the common path copied its P
        // (16 moves per block); tied, the common path keeps 8 64-bit moves.
        PRegs p_new;
        alpha = rescale_block(j, k_cur, s_cur, p_new, ts);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int w = 0; w < 4; ++w)
              p_cur[kt][h][w] = __builtin_amdgcn_update_dpp(p_cur[kt][h][w], p_new[kt][h][w],
                                                            0xE4, 0xF, 0xF, false);
      } else {
        l_run += KVT ? ls * ts.inv_f : ls;
      }
      // O^T holds blocks up to j - 1 now (this iteration's P V has run), all
      // relative to the old reference.  (A branch of its own: inside the one
      // above, the accumulators' rescale next to the matrix instructions there
      // cost the loop ~40 registers.)
      asm volatile("" ::: "memory");
      if (big) {
#pragma unroll
        for (int t = 0; t < NDT; ++t) acc[t] *= alpha;
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NVM) : "memory");
      barrier();
    };
    // Iteration j with j % 4 == 0, 1, 2, 3.
    auto step0 = [&](int j) __attribute__((always_inline)) { step(j, k_lds0, k_lds1, k_lds3, v_lds1, v_lds0, sa, sb, pa, pb); };
    auto step1 = [&](int j) __attribute__((always_inline)) { step(j, k_lds1, k_lds2, k_lds0, v_lds0, v_lds1, sb, sa, pb, pa); };
    auto step2 = [&](int j) __attribute__((always_inline)) { step(j, k_lds2, k_lds3, k_lds1, v_lds1, v_lds0, sa, sb, pa, pb); };
    auto step3 = [&](int j) __attribute__((always_inline)) { step(j, k_lds3, k_lds0, k_lds2, v_lds0, v_lds1, sb, sa, pb, pa); };
    auto last_pv = [&](const uint8_t* vbuf, const PRegs& p_last) __attribute__((always_inline)) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS load outlives the loop
      pv(vbuf, p_last);
      mfma_read_pipeline<NPV, 1, (NPV < 8 ? NPV : 8)>();
    };
    // The loop runs to the next multiple of four blocks: blocks past the last
    // one are fully masked (keys past N, or causal keys after every query of the
    // workgroup), so they change neither m, l nor O.  One copy of the loop body
    // keeps the register allocation of the steady state.
    for (int j = kb_lo; j < kb_hi; j += 4) {
      step0(j);
      step1(j + 1);
      step2(j + 2);
      step3(j + 3);
    }
    last_pv(v_lds1, pb);  // the last iteration is odd: P in pb, V^T in buffer 1
  } else {
    // fp8 P V: V(j+2) goes global -> LDS in iteration j into V stage (j+2)%4,
    // which held V(j-2), read in iteration j-1; P V of block j-1 reads stage
    // (j-1)%4.  Otherwise the iteration is the one above, without the V^T
    // store.  Stage 3 starts zeroed for the P V of the zero block -1 (e4m3
    // bytes 0x7f / 0xff are NaN, and 0 * NaN would be NaN).
    for (int i = tid; i < KBUF / 16; i += kThreads)
      reinterpret_cast<u32x4*>(v_lds3)[i] = u32x4{0u, 0u, 0u, 0u};
    constexpr int NVM8 = 2 * K_PER_W;  // global load instructions per wave per iteration
    load_scales(kb_lo);
    load_k(kb_lo * kBC, k_lds0);
    load_v8(kb_lo * kBC, v_lds0);
    load_k((kb_lo + 1) * kBC, k_lds1);
    load_v8((kb_lo + 1) * kBC, v_lds1);
    load_k((kb_lo + 2) * kBC, k_lds2);
    // This wave's K(0), V(0) and K(1) have landed; V(1) and K(2) may still fly.
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NVM8) : "memory");
    barrier();

    f32x16 sa[2], sb[2];
    P8Regs pa, pb = {};
    pb[8] = 127u;
    qk(k_lds0, sa);
    barrier();

    constexpr int NQK = 2 * NKS;     // QK^T MFMAs per block (one P V MFMA per d tile)
    constexpr int NM8 = NDT + NQK;
    constexpr int VPM8 = (140 + NM8 - 1) / NM8;          // about 140 VALU per block
    constexpr int TPM8 = (kBC / 2 + 1 + NM8 - 1) / NM8;  // kBC / 2 + 1 exponentials
    constexpr int VM08 = (NM8 - NVM8) / 2;
    // The O^T rescale a block's softmax asks for is applied at the top of the
    // next iteration, just before the P V it must precede: a branch after the
    // MFMA run would let the compiler sink that run's QK^T MFMAs behind it.
    bool resc_prev = false;
    float alpha_prev = 1.0f;
    auto step8 = [&](int j, const uint8_t* k_next, uint8_t* k_fill, const uint8_t* v_prev,
                     uint8_t* v_fill, f32x16* s_cur, f32x16* s_next, P8Regs& p_cur,
                     const P8Regs& p_prev) __attribute__((always_inline)) {
      if (needs_mask(j)) mask(s_cur, j * kBC);
      if (resc_prev) {  // O^T still holds blocks up to j-2 only
  #pragma unroll
        for (int t = 0; t < NDT; ++t) acc[t] *= alpha_prev;
      }
      const float sk = sk_next, sv = sv_next;
      load_scales(j + 1);
      load_v8((j + 2) * kBC, v_fill);   // V(j+2)
      load_k((j + 3) * kBC, k_fill);    // K(j+3)
      pv8(v_prev, p_prev);              // P V of block j-1
      qk(k_next, s_next);               // QK^T of block j+1
      alpha_prev = softmax8(s_cur, p_cur, resc_prev, tile_scale(sk, sv));
      mfma_run_pipeline<NDT, 4, NQK, KCH, 2, VPM8, TPM8, 0, NVM8, VM08>();
      // Keep the whole run -- softmax, P V and QK^T MFMAs -- in this block:
      // the compiler would otherwise sink MFMAs past the barrier to their
      // first use in the next iteration.
  #pragma unroll
      for (int i = 0; i < 9; ++i) asm volatile("" ::"v"(p_cur[i]));
      asm volatile("" ::"v"(l_run));
  #pragma unroll
      for (int t = 0; t < NDT; ++t)
  #pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(acc[t][i]));
  #pragma unroll
      for (int kt = 0; kt < 2; ++kt)
  #pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" ::"v"(s_next[kt][i]));
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NVM8) : "memory");
      barrier();
    };
    auto step8_0 = [&](int j) __attribute__((always_inline)) { step8(j, k_lds1, k_lds3, v_lds3, v_lds2, sa, sb, pa, pb); };
    auto step8_1 = [&](int j) __attribute__((always_inline)) { step8(j, k_lds2, k_lds0, v_lds0, v_lds3, sb, sa, pb, pa); };
    auto step8_2 = [&](int j) __attribute__((always_inline)) { step8(j, k_lds3, k_lds1, v_lds1, v_lds0, sa, sb, pa, pb); };
    auto step8_3 = [&](int j) __attribute__((always_inline)) { step8(j, k_lds0, k_lds2, v_lds2, v_lds1, sb, sa, pb, pa); };
    for (int j = kb_lo; j < kb_hi; j += 4) {
      step8_0(j);
      step8_1(j + 1);
      step8_2(j + 2);
      step8_3(j + 3);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no LDS load outlives the loop
    if (resc_prev) {
  #pragma unroll
      for (int t = 0; t < NDT; ++t) acc[t] *= alpha_prev;
    }
    pv8(v_lds3, pb);  // the last iteration is j % 4 == 3: P in pb, V in stage 3
    mfma_read_pipeline<NDT, 4, (NDT < 2 ? NDT : 2)>();
    }

  // ---- epilogue: O = O^T / l (fp16), LSE = ln 2 * (m c + log2 l) ----------------
  const float l_tot = sum_pair32(l_run);
  {
    // O leaves through LDS so that the global stores write whole rows.  The
    // accumulator gives each lane 4-value pieces of one row, so storing it
    // directly scatters every instruction over 32 rows; a wave retires only
    // once its stores have completed, and that held each round of workgroups
    // for microseconds.  Each wave rounds its 32 x D block to fp16 into a K
    // stage (free once every wave has passed the barrier), 16-byte chunks
    // XOR-swizzled by row, reads it back row-major, 16 bytes per lane, and
    // stores whole rows (D consecutive fp16 values in either layout).  One
    // chunk of a split key range stores its rows (O over the chunk's keys) and
    // LSE the same way to its slots of the workspace, for the merge.
    constexpr int OROWB = D * 2;     // bytes of one fp16 row of O
    constexpr int OCH = OROWB / 16;  // 16-byte chunks per row
    constexpr int OWB = kQW * OROWB;  // bytes of one wave's block
    constexpr int WPB = KBUF / OWB;  // waves per K stage
    constexpr int WPV = PV8 ? 0 : VSTAGE / OWB;  // waves per V^T stage (used past the K stages)
    static_assert(WPB >= 1 && kWaves <= 4 * WPB + 2 * WPV, "O staging must fit the K and V stages");
    _Float16* wrows;  // row 0 of this wave's block
    int64_t wstride;  // elements between its rows
    float* wlse;      // LSE of row 0
    if (n_chunks > 1) {
      const int64_t slot0 =
          ((int64_t)(bh * p.n_qtiles + qt) * p.split_cmax + chunk) * kBR + (qw0 - q0);
      wrows = p.ws_o + slot0 * D;
      wstride = D;
      wlse = p.ws_lse + slot0;
    } else {
      wrows = p.o + head_off + (int64_t)qw0 * row_elems;
      wstride = row_elems;
      wlse = p.lse + (int64_t)bh * N + qw0;
    }
    barrier();
    uint8_t* obuf;
    if (wave < 4 * WPB) {
      const int ob = wave / WPB;
      obuf = (ob == 0 ? k_lds0 : ob == 1 ? k_lds1 : ob == 2 ? k_lds2 : k_lds3) + (wave % WPB) * OWB;
    } else {  // fp8 with 8 waves: the K stages hold four waves' blocks, the V^T stages the rest
      constexpr int W = WPV > 0 ? WPV : 1;
      const int vw = wave - 4 * WPB;
      obuf = (vw / W == 0 ? v_lds0 : v_lds1) + (vw % W) * OWB;
    }
    const float inv = __builtin_amdgcn_rcpf(l_tot) * v_scale;  // rows >= N are not stored
#pragma unroll
    for (int t = 0; t < NDT; ++t)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ch = t * 4 + g;  // chunk of d values t*32 + 8g .. +7; this lane's half: 4*hh ..
        u32x2 w = {pack_f16x2(acc[t][4 * g] * inv, acc[t][4 * g + 1] * inv),
                   pack_f16x2(acc[t][4 * g + 2] * inv, acc[t][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(obuf + lr * OROWB + ((ch ^ (lr % OCH)) * 16) + 8 * hh) = w;
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr int RPI = kWave / OCH;  // rows per read instruction
#pragma unroll
    for (int it = 0; it < kQW / RPI; ++it) {
      const int r = it * RPI + lane / OCH, ch = lane % OCH;
      const u32x4 x = *reinterpret_cast<const u32x4*>(obuf + r * OROWB + ((ch ^ (r % OCH)) * 16));
      if (qw0 + r < N) *reinterpret_cast<u32x4*>(wrows + r * wstride + ch * 8) = x;
    }
    const float ref_log2 = PV8 ? ref8 : ref_c;
    if (hh == 0 && my_q < N) wlse[lr] = kLn2 * (ref_log2 + __builtin_amdgcn_logf(l_tot));
  }
}

// ---------------------------------------------------------------------------
// Merge of split key ranges: for each row of a tile whose range was cut into
// chunks, LSE = ln sum_c exp(LSE_c) and O = sum_c exp(LSE_c - LSE) O_c (softmax
// over a union of key sets from the softmaxes over the parts), O rounded to
// fp16.
// ---------------------------------------------------------------------------
struct MergeParams {
  const _Float16* ws_o;
  const float* ws_lse;
  _Float16* o;
  float* lse;
  int N;
  int H;
  int n_qtiles;
  int layout;
  int split_g;
  int split_cmax;
  int causal;
  int qt_lo;  // tiles below it were not split (written directly)
};

constexpr int kMergeEPT = 8;  // d values per merge thread: one 16-byte fp16 load per chunk

// Workgroups of 256 threads the merge launches per query tile of BR rows.
template <int D, int BR>
constexpr int merge_wgs_per_tile() { return BR / (256 / (D / kMergeEPT)); }

template <int D, int BR>
__global__ __launch_bounds__(256) void fa_merge_kernel(MergeParams m) {
  // One thread per row and 8 d values, so every load of a row's chunks is
  // independent and many are in flight: the merge is a pass over the partials
  // at memory speed, 16 bytes per load.
  constexpr int TPR = D / kMergeEPT;  // threads per row
  constexpr int RPW = 256 / TPR;      // rows per workgroup
  constexpr int WPT = BR / RPW;       // workgroups per tile
  static_assert(WPT == merge_wgs_per_tile<D, BR>(), "merge grid");
  const int tile = blockIdx.x / WPT;  // bh * n_qtiles + qt
  const int bh = tile / m.n_qtiles, qt = tile % m.n_qtiles;
  const int groups = m.causal ? qt + 1 : m.n_qtiles;
  const int n = (groups + m.split_g - 1) / m.split_g;
  if (n < 2 || qt < m.qt_lo) return;  // written by an attention kernel itself
  const int r = (blockIdx.x % WPT) * RPW + threadIdx.x / TPR;
  const int row = qt * BR + r;
  if (row >= m.N) return;
  const int e0 = (threadIdx.x % TPR) * kMergeEPT;
  const int64_t slot0 = (int64_t)tile * m.split_cmax * BR + r;  // chunk c: slot0 + c * BR
  float mx = -INFINITY;
  for (int ch = 0; ch < n; ++ch) mx = fmaxf(mx, m.ws_lse[slot0 + (int64_t)ch * BR]);
  float wsum = 0.0f;
  f32x8 acc = {};
#pragma unroll 4
  for (int ch = 0; ch < n; ++ch) {
    const int64_t slot = slot0 + (int64_t)ch * BR;
    const float w = __expf(m.ws_lse[slot] - mx);
    // One 16-byte load converted as a vector (a __builtin_bit_cast of a single
    // element of a loaded vector read element 0 with this compiler).
    const f16x8 x = *reinterpret_cast<const f16x8*>(m.ws_o + slot * D + e0);
    wsum += w;
    acc += w * __builtin_convertvector(x, f32x8);
  }
  const float inv = 1.0f / wsum;
  int64_t off;
  if (m.layout == FA_LAYOUT_BNHD) {
    const int b = bh / m.H, h = bh - b * m.H;
    off = (((int64_t)b * m.N + row) * m.H + h) * D;
  } else {
    off = ((int64_t)bh * m.N + row) * D;
  }
  _Float16* dst = m.o + off + e0;
  *reinterpret_cast<u32x4*>(dst) = u32x4{pack_f16x2(acc[0] * inv, acc[1] * inv),
                                         pack_f16x2(acc[2] * inv, acc[3] * inv),
                                         pack_f16x2(acc[4] * inv, acc[5] * inv),
                                         pack_f16x2(acc[6] * inv, acc[7] * inv)};
  if (e0 == 0) m.lse[(int64_t)bh * m.N + row] = mx + __logf(wsum);
}

// ---------------------------------------------------------------------------
// Host side: argument checks (no HIP calls) and launch.
// ---------------------------------------------------------------------------

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

// Everything but the pointers.
int check_problem(int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
                  int layout, bool* empty) {
  *empty = false;
  if (layout != FA_LAYOUT_BHND && layout != FA_LAYOUT_BNHD) return FA_ERR_LAYOUT;
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
  // One head's rows must stay addressable by 32-bit buffer offsets.
  // B and H are bounded one at a time first, so that B * H cannot overflow.
  if (N > (int64_t)1 << 22 || B > (int64_t)1 << 24 || H > (int64_t)1 << 24 ||
      B * H > (int64_t)1 << 24)
    return FA_ERR_SHAPE;
  // [B, N, H, d]: one head's rows span N*H*d elements.
  const int64_t esize = dtype == FA_DTYPE_FP8_E4M3 ? 1 : 2;
  if (layout == FA_LAYOUT_BNHD && N * H * d * esize > (int64_t)1 << 30) return FA_ERR_SHAPE;
  const int64_t tiles = (N + kMinBR - 1) / kMinBR;
  if (B * H * tiles > INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

int check_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
               int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal, int dtype,
               int layout, bool* empty) {
  const int st = check_problem(B, H, N, d, scale, causal, dtype, layout, empty);
  if (st != FA_OK || *empty) return st;
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_ALIGN;
  return FA_OK;
}

// Query tiles [qt_lo, qt_hi) of every head (tiles of Shape<WAVES>::br rows).
template <int DT, int D, bool CAUSAL, int WAVES, bool PV8 = false, bool KVT = false>
int launch_w(Params prm, int qt_lo, int qt_hi, hipStream_t stream) {
  using S = Shape<WAVES>;
  prm.qt_base = qt_lo;
  prm.n_qtiles = qt_hi - qt_lo;
  void* args[] = {&prm};
  const dim3 grid((unsigned)(prm.bh * prm.n_qtiles));
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(&fa_fwd_kernel<DT, D, CAUSAL, WAVES, PV8, KVT>), grid,
      dim3(S::threads), args, 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

template <int DT, int D, bool CAUSAL, int WAVES>
int launch_all(const Params& prm, hipStream_t stream) {
  return launch_w<DT, D, CAUSAL, WAVES>(prm, 0, (prm.N + Shape<WAVES>::br - 1) / Shape<WAVES>::br,
                                        stream);
}

template <int DT, int D, bool CAUSAL>
int launch_t(const Params& prm, int cus, hipStream_t stream) {
  constexpr int W = default_waves<DT, D>();
  const int64_t wgs8 = (int64_t)prm.bh * ((prm.N + Shape<8>::br - 1) / Shape<8>::br);
  if constexpr (W == 8) {
    // With 256-row tiles filling at most half the CUs, 128-row tiles on all of
    // them finish sooner although one wave per SIMD runs slower than two.
    if (2 * wgs8 <= cus) return launch_all<DT, D, CAUSAL, 4>(prm, stream);
  }
  if constexpr (D == 128 && DT == FA_DTYPE_FP8_E4M3) {
    // fp8 with P V in fp16 converts V to fp16 while staging it: one 8-wave
    // workgroup per CU converts each block once for 256 rows instead of twice
    // for two 128-row tiles (fp8 causal [1,32,16384,128]: 2048 such tiles,
    // 1.74-1.75 -> 1.69-1.70 ms).  With fewer than two 256-row tiles per CU
    // the 128-row tiles balance better (fp8 causal [1,4,16384,128], 256
    // tiles: 0.28 ms, against 0.33 with 8 waves).
    if (wgs8 >= 2 * (int64_t)cus) return launch_all<DT, D, CAUSAL, 8>(prm, stream);
  }
  if constexpr (D == 64 && DT != FA_DTYPE_FP8_E4M3 && CAUSAL) {
    // Causal d = 64 with long tiles on grids of two or more 256-row tiles per
    // CU: 8 waves as well (fp16 [1,8,16384,64] 373 -> 337 us, [2,16,4096,64]
    // 99.5 -> 93.3, bf16 [1,32,8192,64] 348 -> 340, [8,16,4096,64] 384 ->
    // 381).  On fewer tiles the 4-wave workgroups balance the causal tail
    // better ([1,16,4096,64]: 63 us, against 73 with 8 waves), and so they
    // do for short tiles ([2,16,2048,64]: 33.6 against 41.3).
    if (prm.N >= 4096 && wgs8 >= 2 * (int64_t)cus) return launch_all<DT, D, CAUSAL, 8>(prm, stream);
  }
  if constexpr (D == 64 && DT != FA_DTYPE_FP8_E4M3 && !CAUSAL) {
    // Non-causal d = 64 with tiles of 16 or more key blocks: one 8-wave
    // workgroup per CU (one K/V staging for 256 rows) beats three 4-wave ones
    // (fp16 [4,16,1024,64] 26.0 -> 24.9 us, [2,16,4096,64] 178 -> 171 us); with
    // 8 blocks ([16,32,512,64] 53 -> 58 us) or causal tiles the three
    // co-resident 4-wave workgroups hide the per-tile cost better.
    if (prm.N >= 1024 && 2 * wgs8 > cus) return launch_all<DT, D, CAUSAL, 8>(prm, stream);
  }
  return launch_all<DT, D, CAUSAL, W>(prm, stream);
}

// fp8 with P V on the fp8 matrix cores for every query tile whose first row
// sees at least min_keys keys (causal: row i sees i + 1; otherwise all N), and
// in fp16 for the tiles before: two launches over disjoint tiles, both with
// 128-row tiles.
template <int D, bool CAUSAL, bool KVT = false>
int launch_pv8(const Params& prm, int64_t min_keys, hipStream_t stream) {
  constexpr int DT = FA_DTYPE_FP8_E4M3;
  constexpr int BR = Shape<4>::br;
  static_assert(default_waves<DT, D>() == 4, "both launches use 128-row tiles");
  const int n_t = (prm.N + BR - 1) / BR;
  const int64_t mk = min_keys < (int64_t)prm.N + 1 ? min_keys : (int64_t)prm.N + 1;
  int n_lo;  // tiles that keep P V in fp16
  if (CAUSAL)
    n_lo = mk <= 1 ? 0 : (int)((mk - 1 + BR - 1) / BR);  // first row qt*BR sees qt*BR + 1 keys
  else
    n_lo = prm.N >= mk ? 0 : n_t;
  if (n_lo > n_t) n_lo = n_t;
  int st = FA_OK;
  if (n_lo > 0) st = launch_w<DT, D, CAUSAL, 4, false, KVT>(prm, 0, n_lo, stream);
  if (st == FA_OK && n_lo < n_t) st = launch_w<DT, D, CAUSAL, 4, true, KVT>(prm, n_lo, n_t, stream);
  return st;
}

template <int DT>
int launch_dt(const Params& prm, int d, int causal, int cus, hipStream_t stream) {
  if (d == 64)
    return causal ? launch_t<DT, 64, true>(prm, cus, stream)
                  : launch_t<DT, 64, false>(prm, cus, stream);
  return causal ? launch_t<DT, 128, true>(prm, cus, stream)
                : launch_t<DT, 128, false>(prm, cus, stream);
}

// Key-range split for grids that would leave CUs idle or hand the causal tail
// to a few of them.  Work is counted in groups (BR x BR score blocks, BR the
// kernel's tile height): with T tiles per head, causal tile t spans t + 1
// groups and a non-causal one T.  Cutting each tile into ceil(groups / g)
// chunks of at most g groups gives `units` workgroups; with `slots`
// workgroups resident at once (one per CU for 8-wave kernels, two for 4-wave)
// the attention kernel takes about ceil(units / slots) rounds of g + 1/2
// group times (the half for a chunk's prologue and epilogue), and every chunk
// of a split tile adds its partial O and LSE, written and read back once, at
// an effective 5 TB/s.  A group takes 4 BR^2 d FLOP at the slot's share of
// its CU's throughput (kSplitRatePerCU).  Unsplit, the time is the longest tile or
// the work per slot, whichever is larger -- for an 8-wave grid small enough
// to run on the 4-wave twin, with the twin's 128-row tiles (half a group row
// each) at about 0.8 of the 8-wave rate.  The split is taken when estimated
// at least 5 % faster (the estimate has erred on the slow side: shapes
// estimated 5-15 % faster ran 5-9 % faster); grids with at least two tiles
// per slot are left whole (the longest-first order balances them).
// Forward throughput of one CU that the plan assumes, FLOP/s: the whole-grid
// rates the kernels sustain on a 256-CU MI355X under its power limit, divided
// by 256 -- fp16 / bf16 at d = 128 about 1.0 PFLOP/s, fp8 (P V in fp16) about
// 1.3, both at about 0.6 of that at d = 64 (the kernel traces of the default
// workload, the fp8 causal workload and the shapes listed in
// profiles/fa_fwd_workloads_kernel_trace.md).  Only their ratio to the
// partial-result traffic matters, and only roughly.
constexpr double kSplitRatePerCU[2][2] = {  // [fp8][d == 128]
    {0.6e15 / 256, 1.0e15 / 256},
    {0.6 * 1.3e15 / 256, 1.3e15 / 256}};

struct SplitPlan {
  int g = 0;     // chunk size in groups; 0: no split
  int cmax = 0;  // chunks of the longest tile
  int T = 0;     // query tiles per head
  int br = 0;    // rows per tile
  int64_t units = 0;
  int64_t ws_bytes = 0;
};

SplitPlan plan_split(int64_t BH, int64_t N, int64_t d, bool causal, int dtype, int cus) {
  SplitPlan pl;
  const int br = (d == 128 && dtype != FA_DTYPE_FP8_E4M3) ? 256 : 128;  // default_waves * 32
  const int per_cu = br == 256 ? 1 : 2;  // resident workgroups per CU
  const int64_t slots = (int64_t)cus * per_cu;
  const int64_t T = (N + br - 1) / br;
  pl.T = (int)T;
  pl.br = br;
  if (T < 4 || BH * T >= 2 * slots) return pl;
  auto chunks_per_head = [&](int64_t g) {
    if (!causal) return T * ((T + g - 1) / g);
    const int64_t full = T / g, rem = T % g;  // sum over t < T of ceil((t + 1) / g)
    return g * full * (full + 1) / 2 + rem * (full + 1);
  };
  const double rate = kSplitRatePerCU[dtype == FA_DTYPE_FP8_E4M3][d == 128];
  const double t_group = 4.0 * br * br * (double)d / (rate / per_cu);  // seconds
  const double t_partial = 2.0 * br * (2.0 * d + 4.0) / 5e12;  // write + read of a chunk's partial, seconds
  const int64_t total = causal ? BH * T * (T + 1) / 2 : BH * T * T;
  double whole;
  if (br == 256 && 2 * BH * T <= cus) {  // launch_t runs the 4-wave twin
    const double longest = 0.5 * (double)T / 0.8;
    whole = t_group * (causal ? fmax(longest, (double)total / (0.8 * cus)) : longest);
  } else {
    whole = t_group * (causal ? fmax((double)T, (double)((total + slots - 1) / slots))
                              : (double)((BH * T + slots - 1) / slots) * (double)T);
  }
  double best = whole;
  for (int64_t g = T - 1; g >= 1; --g) {  // ties go to fewer, longer chunks
    const int64_t per_head = chunks_per_head(g);
    const int64_t units = BH * per_head;
    // chunks of split tiles: all but the tiles short enough for one chunk
    const int64_t whole_tiles = causal ? (g < T ? g : T) : (g >= T ? T : 0);
    const int64_t split_chunks = BH * (per_head - whole_tiles);
    const double est = (double)((units + slots - 1) / slots) * ((double)g + 0.5) * t_group +
                       (double)split_chunks * t_partial;
    if (est < best) {
      best = est;
      pl.g = (int)g;
    }
  }
  if (pl.g == 0 || best > 0.95 * whole) {
    pl.g = 0;
    return pl;
  }
  pl.cmax = (int)((T + pl.g - 1) / pl.g);
  pl.units = BH * chunks_per_head(pl.g);
  pl.ws_bytes = BH * T * pl.cmax * br * (2 * d + 4);  // O fp16 + LSE fp32 per chunk row
  return pl;
}

// Chunk units of the plan over query tiles [qt_lo, T) (the longest-first
// order lists tiles from T - 1 down, so a shorter count stops above qt_lo).
template <int DT, int D, bool CAUSAL, bool PV8 = false>
int launch_split(Params prm, const SplitPlan& pl, void* ws, hipStream_t stream, int qt_lo = 0) {
  constexpr int W = default_waves<DT, D>();
  using S = Shape<W>;
  prm.n_qtiles = pl.T;
  prm.qt_base = 0;
  prm.split_g = pl.g;
  prm.split_cmax = pl.cmax;
  prm.ws_o = static_cast<_Float16*>(ws);
  prm.ws_lse = reinterpret_cast<float*>(prm.ws_o + (int64_t)prm.bh * pl.T * pl.cmax * S::br * D);
  int64_t units = pl.units;
  if (qt_lo > 0) {  // causal: tile t has ceil((t + 1) / g) chunks
    units = 0;
    for (int t = qt_lo; t < pl.T; ++t) units += (t + pl.g) / pl.g;
    units *= prm.bh;
  }
  void* args[] = {&prm};
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(&fa_fwd_kernel<DT, D, CAUSAL, W, PV8>),
      dim3((unsigned)units), dim3(S::threads), args, 0, stream);
  if (e != hipSuccess) return FA_ERR_LAUNCH;
  MergeParams m;
  m.ws_o = prm.ws_o;
  m.ws_lse = prm.ws_lse;
  m.o = prm.o;
  m.lse = prm.lse;
  m.N = prm.N;
  m.H = prm.H;
  m.n_qtiles = pl.T;
  m.layout = prm.layout;
  m.split_g = pl.g;
  m.split_cmax = pl.cmax;
  m.causal = CAUSAL ? 1 : 0;
  m.qt_lo = qt_lo;
  void* margs[] = {&m};
  constexpr int kMergeWgsPerTile = merge_wgs_per_tile<D, S::br>();
  e = hipLaunchKernel(reinterpret_cast<const void*>(&fa_merge_kernel<D, S::br>),
                      dim3((unsigned)(prm.bh * pl.T * kMergeWgsPerTile)), dim3(256), margs, 0,
                      stream);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

// fp8 P V with the key-range split: tiles whose first row sees fewer than
// min_keys keys run unsplit with fp16 P V (they are short), the others are
// split over the fp8-P V kernel (the whole grid when non-causal and N >=
// min_keys; otherwise fp16 P V split throughout).
template <int D, bool CAUSAL>
int launch_pv8_split(const Params& prm, int64_t min_keys, const SplitPlan& pl, void* ws,
                     hipStream_t stream) {
  constexpr int DT = FA_DTYPE_FP8_E4M3;
  constexpr int BR = Shape<4>::br;
  const int n_t = pl.T;
  const int64_t mk = min_keys < (int64_t)prm.N + 1 ? min_keys : (int64_t)prm.N + 1;
  int n_lo;
  if (CAUSAL)
    n_lo = mk <= 1 ? 0 : (int)((mk - 1 + BR - 1) / BR);
  else
    n_lo = prm.N >= mk ? 0 : n_t;
  if (n_lo > n_t) n_lo = n_t;
  if (n_lo == n_t) return launch_split<DT, D, CAUSAL, false>(prm, pl, ws, stream);
  int st = FA_OK;
  if (n_lo > 0) st = launch_w<DT, D, CAUSAL, 4, false>(prm, 0, n_lo, stream);
  if (st == FA_OK) st = launch_split<DT, D, CAUSAL, true>(prm, pl, ws, stream, n_lo);
  return st;
}

template <int DT>
int launch_split_dt(const Params& prm, int d, int causal, const SplitPlan& pl, void* ws,
                    hipStream_t s) {
  if (d == 64)
    return causal ? launch_split<DT, 64, true>(prm, pl, ws, s)
                  : launch_split<DT, 64, false>(prm, pl, ws, s);
  return causal ? launch_split<DT, 128, true>(prm, pl, ws, s)
                : launch_split<DT, 128, false>(prm, pl, ws, s);
}

// pv8_min_keys < 0: P V in fp16 throughout; otherwise (fp8 only) the split
// of launch_pv8.  split: a plan with g > 0 runs the key-range split with
// workspace ws.
// kv_tiles: per-key-tile K / V scales (fp8 only, no split): P V in fp16
// throughout when pv8_min_keys < 0, else as launch_pv8.
int run(const void* q, const void* k, const void* v, const float* dq, const float* dk,
        const float* dv, void* o, float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
        float scale, int causal, int dtype, int layout, void* stream,
        int64_t pv8_min_keys = -1, const SplitPlan* split = nullptr, void* ws = nullptr,
        bool kv_tiles = false) {
  Params prm;
  prm.q = static_cast<const uint8_t*>(q);
  prm.k = static_cast<const uint8_t*>(k);
  prm.v = static_cast<const uint8_t*>(v);
  prm.descale_q = dq;
  prm.descale_k = dk;
  prm.descale_v = dv;
  prm.o = static_cast<_Float16*>(o);
  prm.lse = lse;
  prm.N = (int)N;
  prm.H = (int)H;
  prm.n_qtiles = 0;  // set per kernel shape at launch
  prm.bh = (int)(B * H);
  prm.layout = layout;
  prm.qt_base = 0;
  prm.scale = scale;
  prm.split_g = 0;
  prm.split_cmax = 0;
  prm.ws_o = nullptr;
  prm.ws_lse = nullptr;
  prm.n_kvt = (int)((N + kBC - 1) / kBC);
  const Topology topo = device_topology();
  prm.n_xcd = topo.xcds;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kv_tiles) {
    constexpr int F8 = FA_DTYPE_FP8_E4M3;
    if (pv8_min_keys >= 0) {
      if (d == 64)
        return causal ? launch_pv8<64, true, true>(prm, pv8_min_keys, s)
                      : launch_pv8<64, false, true>(prm, pv8_min_keys, s);
      return causal ? launch_pv8<128, true, true>(prm, pv8_min_keys, s)
                    : launch_pv8<128, false, true>(prm, pv8_min_keys, s);
    }
    static_assert(default_waves<F8, 64>() == 4 && default_waves<F8, 128>() == 4, "fp8: 4 waves");
    const int n64 = (int)((N + Shape<4>::br - 1) / Shape<4>::br);
    if (d == 64)
      return causal ? launch_w<F8, 64, true, 4, false, true>(prm, 0, n64, s)
                    : launch_w<F8, 64, false, 4, false, true>(prm, 0, n64, s);
    // d = 128: 8-wave workgroups on grids of at least two 256-row tiles per
    // CU, as launch_t chooses for fp8 with per-head scales.
    const int n256 = (int)((N + Shape<8>::br - 1) / Shape<8>::br);
    if ((int64_t)prm.bh * n256 >= 2 * (int64_t)topo.cus)
      return causal ? launch_w<F8, 128, true, 8, false, true>(prm, 0, n256, s)
                    : launch_w<F8, 128, false, 8, false, true>(prm, 0, n256, s);
    return causal ? launch_w<F8, 128, true, 4, false, true>(prm, 0, n64, s)
                  : launch_w<F8, 128, false, 4, false, true>(prm, 0, n64, s);
  }
  if (split && split->g > 0 && dtype == FA_DTYPE_FP8_E4M3 && pv8_min_keys >= 0) {
    if (d == 64)
      return causal ? launch_pv8_split<64, true>(prm, pv8_min_keys, *split, ws, s)
                    : launch_pv8_split<64, false>(prm, pv8_min_keys, *split, ws, s);
    return causal ? launch_pv8_split<128, true>(prm, pv8_min_keys, *split, ws, s)
                  : launch_pv8_split<128, false>(prm, pv8_min_keys, *split, ws, s);
  }
  if (split && split->g > 0) {
    switch (dtype) {
      case FA_DTYPE_FP16: return launch_split_dt<FA_DTYPE_FP16>(prm, (int)d, causal, *split, ws, s);
      case FA_DTYPE_BF16: return launch_split_dt<FA_DTYPE_BF16>(prm, (int)d, causal, *split, ws, s);
      default: return launch_split_dt<FA_DTYPE_FP8_E4M3>(prm, (int)d, causal, *split, ws, s);
    }
  }
  if (dtype == FA_DTYPE_FP8_E4M3 && pv8_min_keys >= 0) {
    if (d == 64)
      return causal ? launch_pv8<64, true>(prm, pv8_min_keys, s)
                    : launch_pv8<64, false>(prm, pv8_min_keys, s);
    return causal ? launch_pv8<128, true>(prm, pv8_min_keys, s)
                  : launch_pv8<128, false>(prm, pv8_min_keys, s);
  }
  switch (dtype) {
    case FA_DTYPE_FP16: return launch_dt<FA_DTYPE_FP16>(prm, (int)d, causal, topo.cus, s);
    case FA_DTYPE_BF16: return launch_dt<FA_DTYPE_BF16>(prm, (int)d, causal, topo.cus, s);
    default: return launch_dt<FA_DTYPE_FP8_E4M3>(prm, (int)d, causal, topo.cus, s);
  }
}

// Split workspace of fa_fwd_kvsplit_noalloc: a file-scope device array, one
// copy per GPU the library runs on, held until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in for
// the symbol); it passes the device address scratch_ptr() looks up.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this GPU's copy of scratch, looked up with
// hipGetSymbolAddress on the first call on each device (with that device
// current) and kept per device; NULL if the runtime refuses.
void* scratch_ptr() {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* ptr = ptrs[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  ptrs[dev].store(ptr, std::memory_order_release);
  return ptr;
}

}  // namespace

extern "C" int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                      int dtype, void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, FA_LAYOUT_BHND, &empty);
  if (st != FA_OK || empty) return st;
  return run(q, k, v, nullptr, nullptr, nullptr, o, lse, B, H, N, d, scale, causal, dtype,
             FA_LAYOUT_BHND, stream);
}

extern "C" int fa_fwd_fp8(const void* q, const void* k, const void* v, const float* descale_q,
                          const float* descale_k, const float* descale_v, void* o, float* lse,
                          int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                          void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, FA_DTYPE_FP8_E4M3,
                      FA_LAYOUT_BHND, &empty);
  if (st != FA_OK || empty) return st;
  if (!descale_q || !descale_k || !descale_v) return FA_ERR_NULL;
  if (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4))
    return FA_ERR_ALIGN;
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal,
             FA_DTYPE_FP8_E4M3, FA_LAYOUT_BHND, stream);
}

extern "C" int fa_fwd_ex(const void* q, const void* k, const void* v, const float* descale_q,
                         const float* descale_k, const float* descale_v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                         int dtype, int layout, void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, layout, &empty);
  if (st != FA_OK || empty) return st;
  if (dtype == FA_DTYPE_FP8_E4M3) {
    const int given = (descale_q != nullptr) + (descale_k != nullptr) + (descale_v != nullptr);
    if (given != 0 && given != 3) return FA_ERR_NULL;
    if (given == 3 &&
        (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4)))
      return FA_ERR_ALIGN;
  } else {
    descale_q = descale_k = descale_v = nullptr;  // not used by fp16 / bf16
  }
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal, dtype,
             layout, stream);
}

extern "C" int fa_fwd_fp8_pv(const void* q, const void* k, const void* v, const float* descale_q,
                             const float* descale_k, const float* descale_v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                             int layout, int64_t min_keys, void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, FA_DTYPE_FP8_E4M3, layout,
                      &empty);
  if (st != FA_OK) return st;
  if (min_keys < 0) return FA_ERR_MIN_KEYS;
  if (empty) return FA_OK;
  const int given = (descale_q != nullptr) + (descale_k != nullptr) + (descale_v != nullptr);
  if (given != 0 && given != 3) return FA_ERR_NULL;
  if (given == 3 && (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4)))
    return FA_ERR_ALIGN;
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal,
             FA_DTYPE_FP8_E4M3, layout, stream, min_keys);
}

extern "C" int fa_fwd_fp8_kvtile(const void* q, const void* k, const void* v,
                                 const float* descale_q, const float* descale_k,
                                 const float* descale_v, void* o, float* lse, int64_t B,
                                 int64_t H, int64_t N, int64_t d, float scale, int causal,
                                 int layout, int64_t pv_min_keys, void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, FA_DTYPE_FP8_E4M3, layout,
                      &empty);
  if (st != FA_OK || empty) return st;
  if (!descale_q || !descale_k || !descale_v) return FA_ERR_NULL;
  if (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4))
    return FA_ERR_ALIGN;
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal,
             FA_DTYPE_FP8_E4M3, layout, stream, pv_min_keys < 0 ? -1 : pv_min_keys, nullptr,
             nullptr, true);
}

extern "C" int64_t fa_fwd_kvsplit_workspace(int64_t B, int64_t H, int64_t N, int64_t d,
                                            int causal, int dtype) {
  bool empty;
  const int st = check_problem(B, H, N, d, 1.0f, causal, dtype, FA_LAYOUT_BHND, &empty);
  if (st != FA_OK) return st;
  if (empty) return 0;
  return plan_split(B * H, N, d, causal != 0, dtype, device_topology().cus).ws_bytes;
}

extern "C" int fa_fwd_kvsplit(const void* q, const void* k, const void* v, const float* descale_q,
                              const float* descale_k, const float* descale_v, void* o, float* lse,
                              int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                              int dtype, int layout, void* workspace, int64_t workspace_bytes,
                              void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, layout, &empty);
  if (st != FA_OK) return st;
  if (workspace_bytes < 0) return FA_ERR_WORKSPACE;
  if (empty) return FA_OK;
  if (dtype == FA_DTYPE_FP8_E4M3) {
    const int given = (descale_q != nullptr) + (descale_k != nullptr) + (descale_v != nullptr);
    if (given != 0 && given != 3) return FA_ERR_NULL;
    if (given == 3 &&
        (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4)))
      return FA_ERR_ALIGN;
  } else {
    descale_q = descale_k = descale_v = nullptr;
  }
  const SplitPlan pl = plan_split(B * H, N, d, causal != 0, dtype, device_topology().cus);
  if (pl.g > 0) {
    if (!workspace) return FA_ERR_NULL;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
    if (workspace_bytes < pl.ws_bytes) return FA_ERR_WORKSPACE;
  }
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal, dtype,
             layout, stream, -1, &pl, workspace);
}

extern "C" int fa_fwd_kvsplit_noalloc(const void* q, const void* k, const void* v,
                                      const float* descale_q, const float* descale_k,
                                      const float* descale_v, void* o, float* lse, int64_t B,
                                      int64_t H, int64_t N, int64_t d, float scale, int causal,
                                      int dtype, int layout, void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, layout, &empty);
  if (st != FA_OK || empty) return st;
  if (dtype == FA_DTYPE_FP8_E4M3) {
    const int given = (descale_q != nullptr) + (descale_k != nullptr) + (descale_v != nullptr);
    if (given != 0 && given != 3) return FA_ERR_NULL;
    if (given == 3 &&
        (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4)))
      return FA_ERR_ALIGN;
  } else {
    descale_q = descale_k = descale_v = nullptr;
  }
  const SplitPlan pl = plan_split(B * H, N, d, causal != 0, dtype, device_topology().cus);
  void* ws = nullptr;
  if (pl.g > 0) {
    if (pl.ws_bytes > kScratchBytes) return FA_ERR_SCRATCH;
    ws = scratch_ptr();
    if (!ws) return FA_ERR_LAUNCH;
  }
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal, dtype,
             layout, stream, -1, &pl, ws);
}

extern "C" int64_t fa_fwd_kvsplit_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int fa_fwd_fp8_pv_kvsplit(const void* q, const void* k, const void* v,
                                     const float* descale_q, const float* descale_k,
                                     const float* descale_v, void* o, float* lse, int64_t B,
                                     int64_t H, int64_t N, int64_t d, float scale, int causal,
                                     int layout, int64_t min_keys, void* workspace,
                                     int64_t workspace_bytes, void* stream) {
  bool empty;
  int st = check_args(q, k, v, o, lse, B, H, N, d, scale, causal, FA_DTYPE_FP8_E4M3, layout,
                      &empty);
  if (st != FA_OK) return st;
  if (min_keys < 0) return FA_ERR_MIN_KEYS;
  if (workspace_bytes < 0) return FA_ERR_WORKSPACE;
  if (empty) return FA_OK;
  const int given = (descale_q != nullptr) + (descale_k != nullptr) + (descale_v != nullptr);
  if (given != 0 && given != 3) return FA_ERR_NULL;
  if (given == 3 && (!aligned(descale_q, 4) || !aligned(descale_k, 4) || !aligned(descale_v, 4)))
    return FA_ERR_ALIGN;
  const SplitPlan pl = plan_split(B * H, N, d, causal != 0, FA_DTYPE_FP8_E4M3,
                                  device_topology().cus);
  if (pl.g > 0) {
    if (!workspace) return FA_ERR_NULL;
    if (!aligned(workspace, 256)) return FA_ERR_ALIGN;
    if (workspace_bytes < pl.ws_bytes) return FA_ERR_WORKSPACE;
  }
  return run(q, k, v, descale_q, descale_k, descale_v, o, lse, B, H, N, d, scale, causal,
             FA_DTYPE_FP8_E4M3, layout, stream, min_keys, &pl, workspace);
}

extern "C" const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "B, H or N is negative or the problem is too large";
    case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case FA_ERR_DTYPE: return "unknown dtype";
    case FA_ERR_ALIGN:
      return "q, k, v, o must be 16-byte aligned (fa_bwd: every pointer), lse and descales "
             "4-byte aligned, a split workspace 256-byte aligned";
    case FA_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case FA_ERR_SCALE: return "scale must be finite and positive";
    case FA_ERR_CAUSAL: return "causal must be 0 or 1";
    case FA_ERR_LAYOUT: return "layout must be FA_LAYOUT_BHND or FA_LAYOUT_BNHD";
    case FA_ERR_MIN_KEYS: return "min_keys must be >= 0";
    case FA_ERR_WORKSPACE: return "workspace smaller than fa_fwd_kvsplit_workspace requires";
    case FA_ERR_SCRATCH:
      return "fa_fwd_kvsplit_noalloc: the split needs more workspace than the library's static "
             "scratch holds (fa_fwd_kvsplit_noalloc_max_bytes); use fa_fwd_kvsplit";
    default: return "unknown status";
  }
}

extern "C" int fa_abi_version(void) { return FA_ABI_VERSION; }
