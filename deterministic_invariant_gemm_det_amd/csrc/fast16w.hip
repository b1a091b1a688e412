// Fast tier, 16-bit inputs: eight waves per workgroup, two per SIMD.
//
// Same arithmetic as fast16.hip, hence the same bits for every
// output element: acc = 0, then acc = V_MFMA_F32_32X32X16_{BF16,F16}(acc,
// A[row, 16s .. 16s+15], B[16s .. 16s+15, col]) for s = 0, 1, ... in order,
// then acc + bias rounded once (sgemm-bi 0.1.2 PyPI page, "Determinism
// contracts"). Only the grouping of outputs into workgroups and the way the
// operands reach the matrix cores differ.
//
// Workgroup: 512 threads = 8 waves in a WR x WC grid over a BM x BN output
// tile; a wave owns (BM / WR) x (BN / WC) outputs as NI x NJ blocks of 32 x 32.
// Two waves share each SIMD, so one wave's matrix-core work covers the other's
// waits. The reduction is walked in stages of 64 indices through two LDS
// slots: while stage s is multiplied out of one slot, stage s + 1 is written
// into the other.
//
// LDS layout of an operand slot: row x holds the stage's 64 reduction indices
// of output row (A) or column (B) x, as eight 16-byte pieces, swizzled so that
// fragment reads (lanes 0..31 rows xb..xb+31 at one piece, lanes 32..63 the
// next piece) spread over the banks. Where one operand is register-transposed
// (the forward weight, dW), rows are paired: pair y = x / 2 occupies 256
// bytes and piece p of row x sits in 16-byte slot (8 (x mod 2) + p) XOR h(y),
// h(y) = ((y XOR y / 8) mod 8) + 8 ((y / 4) mod 2), which also keeps the
// transposing writes apart. Where both operands arrive by direct loads, row x
// occupies 128 bytes with piece p in slot p XOR s(x), s(x) = ((x / 2) mod 8)
// XOR ((x / 8) mod 2): measured on gfx950 with the fragment-read pattern,
// 240 B/clk/CU against 180 for the paired layout, and s has period 32, so a
// lane's fragments of one step are one address plus constants. The slots of
// all stages hold their A regions first, then their B regions.
//
// Filling a slot:
//   * reduction-contiguous source (A of fwd and dX, B of dX): buffer loads that
//     write LDS directly, 1 KB (four row pairs) per wave instruction; lane l
//     fetches the 16-byte source piece that belongs at byte 16 l.
//   * reduction-major source (the forward weight, both operands of dW): a
//     thread loads an 8 x 8 block (8 reduction indices x 8 consecutive
//     columns, eight 16-byte loads) into registers, transposes it with
//     V_PERM_B32 and writes eight 16-byte pieces, one per column. All fragment
//     reads are then plain 16-byte LDS reads.
//
// Applicability (checked on the host): the reduction length is a multiple of
// 64; operands are 16-byte aligned with 16-byte aligned rows; every byte
// offset fits in 31 bits. Pieces past the end of an operand read as zeros
// (buffer range check); rows or columns past the output's edge only reach
// outputs that are never stored.

#include <type_traits>

#include "common.hpp"

namespace detgemm {
namespace w8 {

constexpr int BK_MIN = 64;   // every stage depth is a multiple of this

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

template <typename E> __device__ inline v16f mfma_step(v4u a, v4u b, v16f c);
template <> __device__ inline v16f mfma_step<BF16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}
template <> __device__ inline v16f mfma_step<F16>(v4u a, v4u b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}

// s_waitcnt immediate (gfx9 encoding): at most `vm` vector-memory operations
// outstanding, no LDS operation outstanding, exports unconstrained.
constexpr int waitcnt_vm_lgkm0(int vm) { return (vm & 15) | (7 << 4) | (0 << 8) | (((vm >> 4) & 3) << 14); }

// LDS layouts of an operand region, by stage depth BK (reduction indices per
// stage): row x holds the stage's BK indices of output row (A) or column (B)
// x as BK / 8 pieces of 16 bytes.
template <int BK> struct Lay;

// BK = 64: rows are paired; pair y = x / 2 occupies 256 bytes (all 64 banks
// once) and piece p of row x sits in 16-byte slot (8 (x mod 2) + p) XOR h(y),
// h(y) = ((y XOR y / 8) mod 8) + 8 ((y / 4) mod 2).
template <> struct Lay<64> {
  __host__ __device__ static constexpr int h(int y) { return ((y ^ (y >> 3)) & 7) | (((y >> 2) & 1) << 3); }
  __host__ __device__ static constexpr uint32_t off(int x, int p) {
    return static_cast<uint32_t>((x >> 1) * 256 + 16 * (((x & 1) * 8 + p) ^ h(x >> 1)));
  }
  // The piece that a direct-to-LDS wave instruction gi (1 KB at byte 1024 gi)
  // puts at byte 16 * lane: four row pairs per instruction.
  __device__ static inline void direct(int gi, int lane, int& x, int& p) {
    const int y = 4 * gi + (lane >> 4);
    const int v = (lane & 15) ^ h(y);
    x = 2 * y + (v >> 3);
    p = v & 7;
  }
};

// BK = 64, rows of 128 bytes (used where both operands are staged by direct
// loads): piece p of row x at slot p XOR s(x), s(x) = ((x / 2) mod 8) XOR
// ((x / 8) mod 2). s has period 32 in x, so the fragments of rows x and x + 32
// sit exactly 4096 bytes apart.
struct Lay64r {
  __host__ __device__ static constexpr int sw(int x) { return ((x >> 1) & 7) ^ ((x >> 3) & 1); }
  __host__ __device__ static constexpr uint32_t off(int x, int p) { return static_cast<uint32_t>(x * 128 + 16 * (p ^ sw(x))); }
  __device__ static inline void direct(int gi, int lane, int& x, int& p) {
    x = 8 * gi + (lane >> 3);
    p = (lane & 7) ^ sw(x);
  }
};

// BK = 128: row x occupies 256 bytes and piece p sits in slot p XOR f(x),
// f(x) = (x XOR x / 8) mod 16.
template <> struct Lay<128> {
  __host__ __device__ static constexpr int f(int x) { return (x ^ (x >> 3)) & 15; }
  __host__ __device__ static constexpr uint32_t off(int x, int p) { return static_cast<uint32_t>(x * 256 + 16 * (p ^ f(x))); }
  __device__ static inline void direct(int gi, int lane, int& x, int& p) {
    x = 4 * gi + (lane >> 4);
    p = (lane & 15) ^ f(x);
  }
};

__device__ inline v4u buffer_rsrc(const void* src, int64_t bytes) {
  // base address, stride 0, size in bytes (reads past it return zeros), 32-bit data format
  const uint64_t base = reinterpret_cast<uint64_t>(src);
  return v4u{static_cast<uint32_t>(base), static_cast<uint32_t>(base >> 32) & 0xffffu,
             static_cast<uint32_t>(bytes), 0x00020000u};
}

// Reduction-contiguous operand: element (x, l) at src[x * ld + l]; X rows per
// tile, WAVES waves per workgroup.
template <int X, int WAVES, int BK, typename LAY = Lay<BK>>
struct RcOperand {
  static constexpr int NQ = X * BK * 2 / 1024 / WAVES;   // 1 KB wave instructions per wave per stage
  static_assert(NQ * 1024 * WAVES == X * BK * 2, "tile extent must fill whole wave instructions");
  static constexpr int LOADS = NQ;    // vector-memory instructions per stage per wave
  v4u rsrc;
  uint32_t voff[NQ];   // per-lane source byte offset of instruction q, tile origin 0, stage 0
  uint32_t ld2;        // bytes per source row

  __device__ inline void init(const void* src, int64_t ld, int64_t bytes) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    rsrc = buffer_rsrc(src, bytes);
    ld2 = static_cast<uint32_t>(ld * 2);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      int x, p;
      LAY::direct(wave * NQ + q, lane, x, p);
      voff[q] = static_cast<uint32_t>((x * ld + 8 * p) * 2);
    }
  }
  // Request stage st of the tile whose first row is x0 into the operand slot
  // at `dst`. The loads are inline assembly so that the compiler does not
  // treat them as LDS writes and drain them before unrelated LDS reads;
  // completion is awaited explicitly (vmcnt) before the barrier that publishes
  // the stage. M0 holds the LDS address of the instruction's 1 KB block; the
  // whole byte offset travels in the VGPR operand, so the buffer range check
  // covers every piece.
  __device__ inline void issue(char* dst, int64_t x0, int st) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)dst));
    const uint32_t soff = static_cast<uint32_t>(x0) * ld2 + static_cast<uint32_t>(st) * (BK * 2);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint32_t m0 = lds + 1024u * static_cast<uint32_t>(wave * NQ + q);
      const uint32_t off = voff[q] + soff;
      __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                       :
                       : "s"(m0), "v"(off), "s"(rsrc)
                       : "memory", "m0");
    }
  }
};

// Reduction-major operand: element (x, l) at src[l * ld + x]; X columns per
// tile. Thread t < (64 / KH) (X / 8) owns the KH x 8 block (reduction rows
// KH kb .. KH kb + KH - 1, columns 8 xb .. 8 xb + 7) with kb = t / (X / 8),
// xb = t mod (X / 8): KH 16-byte loads, a V_PERM_B32 transpose, and one
// 2 KH-byte LDS write per column (a whole piece for KH = 8, half of one for
// KH = 4).
template <int X, int KH, int BK>
struct KmOperand {
  static constexpr int NX = X / 8;
  static constexpr int UNITS = (BK / KH) * NX;
  static_assert(X % 64 == 0 && (KH == 4 || KH == 8), "tile extent / block height");
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff;    // byte offset of the thread's block, tile origin 0, stage 0
  uint32_t rstep;   // bytes between reduction rows
  uint32_t sstep;   // bytes between stages
  uint32_t dst;     // the thread's block coordinates, kb | xb << 8
  v4u v[KH];

  __device__ inline bool active() const { return static_cast<int>(threadIdx.x) < UNITS; }

  __device__ inline void init(const void* src, int64_t ld, int64_t bytes) {
    const int t = threadIdx.x;
    const int kb = t / NX, xb = t % NX;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(src), 0, static_cast<int>(bytes), 0x00020000);
    voff = static_cast<uint32_t>((KH * kb * ld + 8 * xb) * 2);
    rstep = static_cast<uint32_t>(ld * 2);
    sstep = static_cast<uint32_t>(BK * ld * 2);
    dst = static_cast<uint32_t>(kb | (xb << 8));
  }
  // Load stage st of the tile whose first column is x0 into registers. The
  // whole byte offset goes into the VGPR operand, so the range check covers it.
  __device__ inline void load(int64_t x0, int st) {
    const uint32_t off = voff + static_cast<uint32_t>(x0) * 2u + static_cast<uint32_t>(st) * sstep;
#pragma unroll
    for (int r = 0; r < KH; ++r)
      v[r] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + static_cast<uint32_t>(r) * rstep, 0, 0);
  }
  // Column c of the block: its KH reduction values packed two per dword.
  __device__ inline void store(char* slot) const {
    const int kb = dst & 0xff, xb = dst >> 8;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      if constexpr (KH == 8) {
        v4u col;
#pragma unroll
        for (int j = 0; j < 4; ++j) col[j] = __builtin_amdgcn_perm(v[2 * j + 1][c >> 1], v[2 * j][c >> 1], sel);
        *reinterpret_cast<v4u*>(slot + Lay<BK>::off(8 * xb + c, kb)) = col;
      } else {
        uint2 col;
        col.x = __builtin_amdgcn_perm(v[1][c >> 1], v[0][c >> 1], sel);
        col.y = __builtin_amdgcn_perm(v[3][c >> 1], v[2][c >> 1], sel);
        *reinterpret_cast<uint2*>(slot + Lay<BK>::off(8 * xb + c, kb >> 1) + 8 * (kb & 1)) = col;
      }
    }
  }
};

// Block height of the register-staged operand: half blocks when there are
// threads for them (fewer registers per thread, more threads sharing the work).
template <int X, int WAVES, int BK> constexpr int km_height() { return (BK / 4) * (X / 8) <= 64 * WAVES ? 4 : 8; }

template <int X, int WAVES, int BK, bool RC> struct OperandOf;
template <int X, int WAVES, int BK> struct OperandOf<X, WAVES, BK, true> { using type = RcOperand<X, WAVES, BK>; };
template <int X, int WAVES, int BK> struct OperandOf<X, WAVES, BK, false> {
  using type = KmOperand<X, km_height<X, WAVES, BK>(), BK>;
  static_assert(type::UNITS <= 64 * WAVES, "register-staged blocks: at most one per thread");
};

// The lane's fragment of the 32-row block at xb for reduction step ks of a
// stage: row xb + lane % 32, piece 2 ks + lane / 32 (elements 16 ks + 8 (lane / 32) + j).
template <int BK>
__device__ inline v4u frag(const char* slot, int xb, int ks) {
  const int lane = threadIdx.x & 63;
  return *reinterpret_cast<const v4u*>(slot + Lay<BK>::off(xb + (lane & 31), 2 * ks + (lane >> 5)));
}

// Output tile t -> (first row, first column). Workgroups are dealt to the
// eight XCDs round-robin, so tile numbers are renumbered to make the tiles
// that run at the same time on one XCD consecutive; consecutive tiles then
// walk G row tiles before the next column tile, so that those tiles share A
// rows and B columns in the XCD's L2.
template <int BM, int BN>
__device__ inline void tile_origin(const GemmArgs& a, uint32_t t, int64_t& row0, int64_t& col0) {
  const uint32_t ntr = static_cast<uint32_t>((a.rows + BM - 1) / BM);
  const uint32_t ntc = static_cast<uint32_t>((a.cols + BN - 1) / BN);
  const uint32_t ntiles = ntr * ntc;
  if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
  constexpr uint32_t G = 4;
  const uint32_t grp = t / (G * ntc), first = grp * G;
  const uint32_t gsz = ntr - first < G ? ntr - first : G;
  const uint32_t within = t - grp * G * ntc;
  row0 = static_cast<int64_t>(first + within % gsz) * BM;
  col0 = static_cast<int64_t>(within / gsz) * BN;
}

// One output tile per workgroup.
//
// Matrix-core operand order: each 32 x 32 block is computed transposed,
// acc = MFMA(B fragment, A fragment, acc), so that a lane holds one output
// row and four consecutive output columns per group of four accumulators.
// Each output element still receives the same 16 products per instruction,
// in the same instruction order.
//
// Reduction steps (16 indices each, four per stage) run in one sequence; the
// fragments of step t + 2 are read from LDS while step t's MFMAs run (four
// fragment buffers, step t in buffer t mod 4; one read placed after each
// matrix instruction). Stage g + 1 must therefore be
// visible before step 4 g + 2 reads it: between steps 4 g + 1 and 4 g + 2 each
// wave writes its register-staged part of the last requested stage, waits for
// its own loads of stage g + 1, and meets the others at a barrier. After the
// barrier every wave has read all of stage g (steps 4 g + 2 and 4 g + 3 are
// already in registers), so stage g + NS is requested into its slot.
//
// Epilogue: acc + bias, one rounding, written through LDS (the stage slots are
// free by then) as a row-major tile, then copied out with 16-byte stores
// along whole tile rows.
template <typename E, bool A_RC, bool B_RC, int BM, int BN, int WR, int WC, int NS, int BK, int WPE>
__global__ void __launch_bounds__(64 * WR * WC, WPE) fast16w_kernel(GemmArgs args) {
  using T = typename E::T;
  constexpr int WAVES = WR * WC, THREADS = 64 * WAVES;
  constexpr int WM = BM / WR, WN = BN / WC, NI = WM / 32, NJ = WN / 32;
  static_assert((WAVES == 8 || WAVES == 4) && NI * 32 == WM && NJ * 32 == WN, "bad wave grid");
  constexpr int KS = BK / 16;   // reduction steps per stage
  static_assert(KS % 4 == 0, "whole groups of four reduction steps per stage");
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, SLOT = A_BYTES + B_BYTES;
  constexpr int RS = BN * 2 + 16;   // LDS row stride of the output tile (bytes)
  static_assert(BM * RS <= NS * SLOT, "output tile must fit the stage slots");
  constexpr int WG_PER_CU = WPE * 4 / WAVES < 1 ? 1 : WPE * 4 / WAVES;
  static_assert(NS >= 2 && NS * SLOT * WG_PER_CU <= 160 * 1024, "LDS of the resident workgroups");
  // direct-to-LDS loads per wave per stage (the ones vmcnt must account for)
  constexpr int DL = (A_RC ? RcOperand<BM, WAVES, BK>::LOADS : 0) + (B_RC ? RcOperand<BN, WAVES, BK>::LOADS : 0);
  static_assert((NS - 2) * DL <= 63 && NS <= 4, "vmcnt range; the stage wait below handles up to four stages");
  constexpr bool KM = !A_RC || !B_RC;
  __shared__ __attribute__((aligned(1024))) char lds[NS * SLOT];

  // Tile and, for a split reduction, chunk of this workgroup: chunk c covers
  // stages s0 .. s0 + nst - 1 and writes f32 partials instead of the output.
  const uint32_t ntiles = static_cast<uint32_t>(((args.rows + BM - 1) / BM) * ((args.cols + BN - 1) / BN));
  uint32_t tb = blockIdx.x;
  int chunk = 0;
  if (args.partial) {
    chunk = static_cast<int>(tb / ntiles);
    tb -= static_cast<uint32_t>(chunk) * ntiles;
  }
  int64_t row0, col0;
  tile_origin<BM, BN>(args, tb, row0, col0);
  const int nst_all = static_cast<int>(args.red / BK);
  const int s0 = args.partial ? chunk * args.chunk_stages : 0;
  const int nst = args.partial ? (nst_all - s0 < args.chunk_stages ? nst_all - s0 : args.chunk_stages) : nst_all;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int wm = (wave / WC) * WM;
  const int wn = (wave % WC) * WN;

  // both operands staged by direct loads in stages of 64: the periodic layout,
  // whose fragment offsets are a per-lane value per step plus constants
  constexpr bool RR = A_RC && B_RC && BK == 64;
  std::conditional_t<RR, RcOperand<BM, WAVES, BK, Lay64r>, typename OperandOf<BM, WAVES, BK, A_RC>::type> oa;
  std::conditional_t<RR, RcOperand<BN, WAVES, BK, Lay64r>, typename OperandOf<BN, WAVES, BK, B_RC>::type> ob;
  oa.init(args.A, args.lda, args.a_bytes);
  ob.init(args.B, args.ldb, args.b_bytes);
  const bool has_bias = args.bias != nullptr;

  // LDS: the A regions of the NS stage slots, then their B regions (a
  // slot's base is then a constant offset of each fragment read)
  auto region_a = [&](int sl) { return lds + sl * A_BYTES; };
  auto region_b = [&](int sl) { return lds + NS * A_BYTES + sl * B_BYTES; };
  // Everything stage st needs from global memory: the register-staged
  // operand first, then the direct-to-LDS ones (so that waiting for the
  // latter covers the former).
  auto request = [&](int st) {
    if constexpr (!A_RC) { if (oa.active()) oa.load(row0, s0 + st); }
    if constexpr (!B_RC) { if (ob.active()) ob.load(col0, s0 + st); }
    if constexpr (A_RC) oa.issue(region_a(st % NS), row0, s0 + st);
    if constexpr (B_RC) ob.issue(region_b(st % NS), col0, s0 + st);
  };
  auto write_km = [&](int st) {
    if constexpr (!A_RC) { if (oa.active()) oa.store(region_a(st % NS)); }
    if constexpr (!B_RC) { if (ob.active()) ob.store(region_b(st % NS)); }
  };
  // per-lane fragment offsets of each step of a stage (periodic layout: the
  // fragments 32 rows further sit 4096 bytes further)
  constexpr bool PRE = RR;
  uint32_t fa[PRE ? KS : 1], fb[PRE ? KS : 1];
  if constexpr (PRE) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fa[ks] = Lay64r::off(wm + (lane & 31), 2 * ks + (lane >> 5));
      fb[ks] = Lay64r::off(wn + (lane & 31), 2 * ks + (lane >> 5));
    }
  }
  // fragments of step ks of the stage in slot sl
  auto read_step = [&](v4u (&af)[NI], v4u (&bf)[NJ], int sl, int ks) {
    const char* As = lds + sl * A_BYTES;
    const char* Bs = lds + NS * A_BYTES + sl * B_BYTES;
    if constexpr (PRE) {
      // one address per operand and step; the fragments 32 rows apart at immediate offsets
      const char* pa = As + fa[ks];
      const char* pb = Bs + fb[ks];
#pragma unroll
      for (int i = 0; i < NI; ++i) af[i] = *reinterpret_cast<const v4u*>(pa + 4096 * i);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = *reinterpret_cast<const v4u*>(pb + 4096 * j);
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) af[i] = frag<BK>(As, wm + 32 * i, ks);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[j] = frag<BK>(Bs, wn + 32 * j, ks);
    }
  };

  // Prologue: stages 0 .. NS - 1 requested and stage 0 published; the last
  // requested stage may still be in flight (its register-staged part is then
  // written before the first barrier of the loop).
  int pending = -1;    // stage whose register-staged part is still in registers
  const int pro = nst < NS ? nst : NS;
  if constexpr (KM) {
    // the registers hold one stage: complete stages one by one, leave the last one pending
    for (int st = 0; st + 1 < pro; ++st) {
      request(st);
      __builtin_amdgcn_s_waitcnt(0);
      __asm__ volatile("" ::: "memory");
      write_km(st);
    }
    request(pro - 1);
    if (pro == 1) {
      __builtin_amdgcn_s_waitcnt(0);
      __asm__ volatile("" ::: "memory");
      write_km(0);
    } else {
      pending = pro - 1;
    }
  } else {
    for (int st = 0; st < pro; ++st) request(st);
    // stage 0 landed; the direct loads of stages 1 .. pro - 1 may still fly
    if (pro == NS) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0((NS - 1) * DL));
    else __builtin_amdgcn_s_waitcnt(0);
  }
  int requested = pro;   // stages requested so far
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");

  v16f acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  v4u af[4][NI], bf[4][NJ];
  read_step(af[0], bf[0], 0, 0);
  read_step(af[1], bf[1], 0, 1);

  // One stage of the sequence. The last stage is a separate copy (LAST), so
  // that the loop body has no branch around the barrier and the next stage's
  // fragment reads: the compiler's LDS wait counts then stay exact.
  // The tile's bias slice goes into the LDS slot that stage nst - 2 used
  // (free from the start of the last stage on; an unused slot when nst < NS)
  // by one direct load at the start of the last stage.
  char* const bias_lds = region_a((nst + NS - 2) % NS);
  static_assert(BN * 2 <= 1024, "bias slice must fit one wave instruction");
  auto load_bias = [&]() {
    if (wave == 0 && lane < BN * 2 / 16) {
      const v4u brsrc = buffer_rsrc(args.bias, args.cols * 2);
      const uint32_t dst = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)bias_lds));
      const uint32_t off = static_cast<uint32_t>(col0) * 2u + 16u * static_cast<uint32_t>(lane);
      __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                       :
                       : "s"(dst), "v"(off), "s"(brsrc)
                       : "memory", "m0");
    }
  };
  auto stage = [&](int g, auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const int SL = g % NS, SLN = (g + 1) % NS;
    if constexpr (LAST) { if (has_bias) load_bias(); }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks == KS - 2 && !LAST) {
        if constexpr (KM) {
          if (pending >= 0) {
            // outstanding after the register-staged loads: that stage's direct loads
            __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(DL));
            __asm__ volatile("" ::: "memory");
            write_km(pending);
            pending = -1;
          }
        }
        // stage g + 1 landed: issued after its loads are only the direct loads
        // of the stages requested after it, g + 2 .. requested - 1 (NS - 2 of
        // them in the steady state, fewer near the end of the reduction)
        {
          const int after = requested - (g + 2);
          if (NS >= 4 && after >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * DL));
          else if (NS >= 3 && after >= 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(DL));
          else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        }
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __asm__ volatile("" ::: "memory");
        if (requested < nst) {
          request(requested);
          if constexpr (KM) pending = requested;
          ++requested;
        }
      }
      // fragments of step 4 g + ks + 2
      if (ks < KS - 2) read_step(af[(ks + 2) & 3], bf[(ks + 2) & 3], SL, ks + 2);
      else if (!LAST) read_step(af[(ks + 2) & 3], bf[(ks + 2) & 3], SLN, ks + 2 - KS);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = mfma_step<E>(bf[ks & 3][j], af[ks & 3][i], acc[i][j]);
      // one fragment read of step ks + 2 after each matrix instruction of step ks
#pragma unroll
      for (int t = 0; t < NI + NJ && t < NI * NJ; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if constexpr (NI * NJ > NI + NJ) __builtin_amdgcn_sched_group_barrier(0x008, NI * NJ - (NI + NJ), 0);
    }
  };
  for (int g = 0; g + 1 < nst; ++g) stage(g, std::false_type{});
  stage(nst - 1, std::true_type{});

  const int lr = lane & 31, lh = lane >> 5;
  if (args.partial || args.out_f32) {
    // split reduction: this chunk's f32 partials; f32 output: the accumulators
    // themselves (no bias in dW); 16 bytes (4 columns) per store
    float* __restrict__ P = args.partial ? args.partial + static_cast<int64_t>(chunk) * args.rows * args.cols
                                         : static_cast<float*>(args.out);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t row = row0 + wm + 32 * i + lr;
      if (row >= args.rows) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t col = col0 + wn + 32 * j + 8 * q + 4 * lh;
          float* y = P + row * args.cols + col;
          if (col + 4 <= args.cols) {
            *reinterpret_cast<v4u*>(y) = v4u{__float_as_uint(acc[i][j][4 * q]), __float_as_uint(acc[i][j][4 * q + 1]),
                                            __float_as_uint(acc[i][j][4 * q + 2]), __float_as_uint(acc[i][j][4 * q + 3])};
          } else {
            for (int e = 0; e < 4 && col + e < args.cols; ++e) y[e] = acc[i][j][4 * q + e];
          }
        }
    }
    return;
  }

  // Epilogue. Every wave is done with the stage slots after this barrier.
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  // the lane's bias values (columns wn + 32 j + 8 q + 4 (lane / 32) + e), read
  // before the output tile overwrites the slot that holds them
  uint2 bias_raw[NJ][4];
  if (has_bias) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        bias_raw[j][q] = *reinterpret_cast<const uint2*>(bias_lds + 2 * (wn + 32 * j + 8 * q + 4 * lh));
    __builtin_amdgcn_s_waitcnt(0);
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // the lane's 4 columns: wn + 32 j + 8 q + 4 (lane / 32) + e of the tile
      const int cl = wn + 32 * j + 8 * q + 4 * lh;
      float b[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (has_bias) {
        const uint2 raw = bias_raw[j][q];
        const T* bt = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int e = 0; e < 4; ++e) b[e] = E::to_f32(bt[e]);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        uint16_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float r = acc[i][j][4 * q + e];
          if (has_bias) r = r + b[e];
          v[e] = __builtin_bit_cast(uint16_t, round_from_f32<E>(r));
        }
        uint2 w;
        w.x = static_cast<uint32_t>(v[0]) | (static_cast<uint32_t>(v[1]) << 16);
        w.y = static_cast<uint32_t>(v[2]) | (static_cast<uint32_t>(v[3]) << 16);
        *reinterpret_cast<uint2*>(lds + (wm + 32 * i + lr) * RS + 2 * cl) = w;
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
  // copy-out: 16-byte chunk u of the tile is row u / (BN / 8), columns 8 (u mod (BN / 8)) ..
  constexpr int CPR = BN / 8;
  T* __restrict__ Y = static_cast<T*>(args.out);
  const bool wide = (args.cols % 8) == 0 && (reinterpret_cast<uintptr_t>(args.out) % 16) == 0;
#pragma unroll 4
  for (int u = threadIdx.x; u < BM * CPR; u += THREADS) {
    const int r = u / CPR, c = u - r * CPR;
    const int64_t row = row0 + r, col = col0 + 8 * c;
    if (row >= args.rows || col >= args.cols) continue;
    const v4u val = *reinterpret_cast<const v4u*>(lds + r * RS + 16 * c);
    T* y = Y + row * args.cols + col;
    if (wide && col + 8 <= args.cols) {
      *reinterpret_cast<v4u*>(y) = val;
    } else {
      const T* vt = reinterpret_cast<const T*>(&val);
      for (int e = 0; e < 8 && col + e < args.cols; ++e) y[e] = vt[e];
    }
  }
}

template <typename E, bool AC, bool BC, int BM, int BN, int WR, int WC, int NS, int BK = 64, int WPE = 8 / (WR * WC)>
hipError_t launch_typed(const GemmArgs& a, hipStream_t stream) {
  // a split reduction counts its chunks in stages of 64
  if (a.red % BK != 0 || (a.partial && BK != 64)) return hipErrorInvalidValue;
  const int64_t tiles = ((a.cols + BN - 1) / BN) * ((a.rows + BM - 1) / BM);
  // one tile (and reduction chunk) per workgroup: a workgroup's stores then
  // overlap the start of the next workgroup on its compute unit
  const int64_t grid = tiles * (a.partial ? a.split : 1);
  // the kernel counts tiles and (tile, stage) pairs in 32 bits
  if (grid > 0x7fffffff || a.red / BK > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fast16w_kernel<E, AC, BC, BM, BN, WR, WC, NS, BK, WPE>), dim3(static_cast<unsigned>(grid)), dim3(64 * WR * WC),
                     0, stream, a);
  return hipGetLastError();
}

// Tile shape from the output's column count only (never from the row count,
// which for fwd and dX is the batch): 256 x 192 for wide outputs, 128 x 192
// for narrow ones, so that an 8192-row batch gives whole rounds of tiles on
// 256 compute units in both cases.
template <typename E, bool AC, bool BC>
hipError_t launch_shape(const GemmArgs& a, int shape, hipStream_t stream) {
  switch (shape) {
    case 0: return launch_typed<E, AC, BC, 256, 192, 4, 2, 2>(a, stream);
    case 1: return launch_typed<E, AC, BC, 128, 192, 4, 2, 2>(a, stream);
    case 2: return launch_typed<E, AC, BC, 128, 192, 2, 2, 2>(a, stream);   // four waves, two workgroups per CU
    case 3: return launch_typed<E, AC, BC, 64, 192, 2, 2, 2>(a, stream);    // four waves, two workgroups per CU
    case 5: return launch_typed<E, AC, BC, 256, 192, 2, 2, 2, 64, 1>(a, stream);   // four waves of 128 x 96, one per SIMD
    default:   // stages of 128 (half the barriers) where the reduction allows it
      if (a.red % 128 != 0 || a.partial) return launch_typed<E, AC, BC, 128, 192, 4, 2, 2>(a, stream);
      return launch_typed<E, AC, BC, 128, 192, 4, 2, 2, 128>(a, stream);
  }
}

template <typename E>
hipError_t launch_op(Op op, const GemmArgs& a, int shape, hipStream_t stream) {
  switch (op) {
    case OP_FWD: return launch_shape<E, true, false>(a, shape, stream);   // X[i][k], W[k][j]
    case OP_DX:  return launch_shape<E, true, true>(a, shape, stream);    // dY[i][n], W[q][n]
    case OP_DW:  return launch_shape<E, false, false>(a, shape, stream);  // X[i][q], dY[i][j]
  }
  return hipErrorInvalidValue;
}

// Ordered combine of a split reduction: out = round(((P_0 + P_1) + ...) +
// P_{S-1}) element by element, f32 additions in ascending chunk order, eight
// elements per thread.
template <typename E>
__global__ void __launch_bounds__(256) combine_kernel(const float* __restrict__ P, int split, int64_t count,
                                                      typename E::T* __restrict__ out, bool vec) {
  using T = typename E::T;
  static_assert(sizeof(T) == 2 || sizeof(T) == 4, "16- or 32-bit output");
  const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i0 >= count) return;
  if (vec && i0 + 8 <= count) {
    float acc[8];
    const v4u a0 = *reinterpret_cast<const v4u*>(P + i0), a1 = *reinterpret_cast<const v4u*>(P + i0 + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) { acc[e] = __uint_as_float(a0[e]); acc[4 + e] = __uint_as_float(a1[e]); }
    for (int c = 1; c < split; ++c) {
      const float* Pc = P + static_cast<int64_t>(c) * count + i0;
      const v4u b0 = *reinterpret_cast<const v4u*>(Pc), b1 = *reinterpret_cast<const v4u*>(Pc + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) { acc[e] = acc[e] + __uint_as_float(b0[e]); acc[4 + e] = acc[4 + e] + __uint_as_float(b1[e]); }
    }
    if constexpr (sizeof(T) == 2) {
      uint16_t v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(uint16_t, round_from_f32<E>(acc[e]));
      v4u w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = static_cast<uint32_t>(v[2 * e]) | (static_cast<uint32_t>(v[2 * e + 1]) << 16);
      *reinterpret_cast<v4u*>(out + i0) = w;
    } else {
      *reinterpret_cast<v4u*>(out + i0) = v4u{__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]), __float_as_uint(acc[3])};
      *reinterpret_cast<v4u*>(out + i0 + 4) = v4u{__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]), __float_as_uint(acc[7])};
    }
    return;
  }
  for (int64_t i = i0; i < i0 + 8 && i < count; ++i) {
    float acc = P[i];
    for (int c = 1; c < split; ++c) acc = acc + P[static_cast<int64_t>(c) * count + i];
    out[i] = round_from_f32<E>(acc);
  }
}

}  // namespace w8

hipError_t launch_combine(Dt dt, bool out_f32, const float* partial, int split, int64_t count, void* out,
                          hipStream_t stream) {
  const int64_t blocks = (count + 256 * 8 - 1) / (256 * 8);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool vec = count % 4 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (out_f32)
    hipLaunchKernelGGL(w8::combine_kernel<F32>, grid, block, 0, stream, partial, split, count, static_cast<float*>(out), vec);
  else if (dt == DT_BF16)
    hipLaunchKernelGGL(w8::combine_kernel<BF16>, grid, block, 0, stream, partial, split, count, static_cast<uint16_t*>(out), vec);
  else if (dt == DT_F16)
    hipLaunchKernelGGL(w8::combine_kernel<F16>, grid, block, 0, stream, partial, split, count, static_cast<_Float16*>(out), vec);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

bool fast16_w_ok(const GemmArgs& a) {
  return a.red % w8::BK_MIN == 0 && a.vec_a && a.vec_b && a.off32_a && a.off32_b &&
         reinterpret_cast<uintptr_t>(a.bias) % 16 == 0;
}

// Wide outputs: 256 x 192 tiles, except long reductions (4096 indices or
// more) into at most 4096 columns, which measured faster as 128 x 192 tiles
// in two four-wave workgroups per compute unit; narrow outputs: 128 x 192
// tiles with stages of 128 reduction indices where the reduction allows it
// (shape 4 falls back to stages of 64 otherwise). Chosen from the column count
// and the reduction length only, never the row count.
int fast16_w_shape(int64_t cols, int64_t red) {
  if (cols < 1536) return 4;
  return (red >= 4096 && cols <= 4096) ? 2 : 0;
}

// dW with dY supplied transposed ([n][m], contiguous along the reduction) and x
// as given (reduction-major): 256 x 192 tiles.
hipError_t launch_fast16_w_dw_bt(Dt dt, const GemmArgs& a, int shape, hipStream_t stream) {
  if (shape == 5) {
    if (dt == DT_BF16) return w8::launch_typed<BF16, false, true, 256, 192, 2, 2, 2, 64, 1>(a, stream);
    if (dt == DT_F16) return w8::launch_typed<F16, false, true, 256, 192, 2, 2, 2, 64, 1>(a, stream);
    return hipErrorInvalidValue;
  }
  if (dt == DT_BF16) return w8::launch_typed<BF16, false, true, 256, 192, 4, 2, 2>(a, stream);
  if (dt == DT_F16) return w8::launch_typed<F16, false, true, 256, 192, 4, 2, 2>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_fast16_w(Op op, Dt dt, const GemmArgs& a, int shape, hipStream_t stream) {
  if (dt == DT_BF16) return w8::launch_op<BF16>(op, a, shape, stream);
  if (dt == DT_F16) return w8::launch_op<F16>(op, a, shape, stream);
  return hipErrorInvalidValue;
}

}  // namespace detgemm
