// Fused tile-group precision-routed prefill attention for gfx950 (TileMix paper, Sections 4.1
// and 4.3): for each query tile the kernel streams key/value tiles, decodes one route bit per
// key-tile group from the packed word of its (KV head, query-tile row) (Section 4.2 lookup
// equation), computes the score tile with the FP16 or the INT8 matrix-core path, and feeds both
// into one fp32 online-softmax state (Section 3.1 recurrence) before an FP16 P.V.
//
// Work decomposition
//   * one workgroup = 8 wavefronts (two per SIMD) = 256 query rows of one query head of one
//     sequence; grid = (query heads, query tiles in reverse order, sequences). Heads vary
//     fastest and are ordered so that consecutive workgroups (which the hardware deals out to
//     the 8 XCDs in turn) keep the query heads of one KV head on one XCD and its L2, and the
//     heaviest causal tiles start first. With a multiple of 8 KV heads and 64 or more query
//     tiles, each XCD instead works through its KV heads one at a time (all query tiles of one,
//     heaviest first, then the next), so that the workgroups in flight on an XCD share one KV
//     head's tiles in its L2 rather than several; with one KV head per XCD (8 KV heads) the two
//     orders are the same. On the V^T path the kernel is launched persistent: as many workgroups
//     as the device holds, taking these work items from per-XCD queues (see prefill_fwd_kernel),
//     so that the XCDs, which run at slightly different speeds, finish together.
//   * each wavefront owns 32 query rows and computes TRANSPOSED score tiles S^T = K Q^T with
//     32x32 MFMAs, so the accumulator lands in the B-operand layout of O^T += V^T P^T: lane l
//     holds query l%32. Key rows inside each 32-key block are loaded in a permuted order (bits 2
//     and 3 of the row index swapped) so that accumulator slots t = 0..7 and 8..15 of lane l
//     hold 8 CONSECUTIVE keys each: key = 32*kb + 16*(t>>3) + 8*(l>>5) + (t&7).
//   * the route bit of a key tile is uniform over each wavefront (route tiles are multiples of
//     32 rows and 64 keys), so the FP16 / INT8 choice is a wave-uniform branch.
//
// Schedule (per wavefront, one 64-key tile per iteration)
//   After the tile's barrier each wavefront reads all K fragments of the tile and issues the
//   score MFMAs of both 32-key halves (two interleaved accumulator chains), reads the per-key
//   factors and converts the scores, then exponentiates both halves (VALU) with the P.V MFMAs
//   of the PREVIOUS tile (its V fragments and P kept from the last iteration) issued among
//   those instructions, so that the wavefront's own matrix-core work overlaps its softmax; one
//   slow-path check per tile follows. P alternates between two register sets and V keeps three
//   LDS stages (tiles n-1, n, n+1); the last tile's P.V follows the loop. Operand reads
//   are issued ahead of their MFMAs so that each waits only for its own data: the direct loads
//   are written as inline assembly, because the compiler counts a pending direct load against
//   the LDS counter too and would then wait for every LDS read to finish before each MFMA. One
//   barrier per 64-key tile; the next tile's K (fp16 and/or int8, as the route bits of the
//   workgroup ask), V and per-key factors are fetched with direct global->LDS loads while the
//   current tile is computed. The queries never pass through LDS: each lane keeps its row's fp16
//   fragments (the FP16 route's B operand, 32 registers at head_dim 128) and int8 fragments in
//   registers, which leaves LDS to the K / V / factor stages (96.5 KiB at head_dim 128).
//
// V: two paths, bitwise the same results. V^T path: a pre-pass writes every 64-key tile of V
//   transposed and chunk-swizzled, the kernel streams it as contiguous 1 KiB blocks and reads
//   each P.V operand fragment with one 16-byte LDS read. Direct path (no pre-pass): the kernel
//   stages V rows as they are (chunk-swizzled on the load side) and builds each operand fragment
//   with two transposing 8-byte LDS reads (ds_read_b64_tr_b16), twice the LDS read instructions.
//   The host picks the direct path when the pre-pass would cost more than those reads, i.e. for
//   short sequences.
//
// Softmax
//   Base 2, with the score scale folded into one FMA per element. The running max is only
//   raised when needed: each tile is exponentiated against the current max, and only if some
//   lane's sum of P over the tile exceeds 2^15 (so that no P can overflow fp16) or the row has
//   no max yet (the wavefront's first tile) does the wavefront take the slow path, which takes
//   the true max, rescales O and l and recomputes P. The row sum is taken from the fp16-rounded
//   P that also feeds P.V (one running sum over both key halves of a tile) and is kept per lane
//   half until the epilogue. P is assembled from packed fp16 pairs (32-bit words), so that the
//   slow path's join merges whole registers instead of re-packing halves.
//
// INT8 scores
//   The int32 accumulator is converted to fp32 and multiplied by the key's k_scale (staged per
//   tile from k_scale with one 4-byte direct load per lane), then one FMA with the per-row factor and the running max gives
//   the exponent. The scales reach the multiply through a DPP row broadcast: each lane loads one
//   scale per 32-key half and accumulator slot t takes it from lane t of its 16-lane row.
#include <type_traits>
#include <utility>

#include "device_types.h"
#include "launch.h"
#include "tile_layout.h"

namespace tilemix {
namespace {

constexpr int BN = kKeyTile;  // keys per pipeline tile
constexpr int NW = 8;         // wavefronts per workgroup
constexpr int ROWS_W = 32;    // query rows per wavefront
constexpr int BM = NW * ROWS_W;
constexpr float P_LIMIT = 32768.0f;  // fast path: a lane's sum of P over a tile stays below this

// LDS layout. Rows are unpadded; 16-byte chunks are XOR-swizzled per row so that each 1 KiB
// block stays contiguous (one direct wave load) while the rows one operand read touches fall in
// distinct banks.
template <int D>
struct Smem {
  static constexpr int RB16 = D * 2;  // bytes per fp16 row of K
  static constexpr int RB8 = D;       // bytes per int8 row of K8
  static constexpr int C16 = RB16 / 16;
  static constexpr int C8 = RB8 / 16;
  static constexpr int KBUF = 0;                  // two K stages
  static constexpr int K16 = 0;                   // offsets inside one K stage
  static constexpr int K8 = K16 + BN * RB16;
  static constexpr int KSTAGE = K8 + BN * RB8;
  static constexpr int VBUF = KBUF + 2 * KSTAGE;  // three V stages: [BN keys][D] fp16 rows (direct
                                                  // path) or [D][BN] V^T as vt_pack.hip writes it
  static constexpr int RBV = D * 2;               // bytes per V row
  static constexpr int CV = RBV / 16;
  static constexpr int VSTAGE = BN * RBV;
  static constexpr int SBUF = VBUF + 3 * VSTAGE;  // two slots of per-key factors
  static constexpr int SSLOT = BN * 4;            // k_scale of the tile's keys
  static constexpr int BYTES = SBUF + 2 * SSLOT;
  // The 16 lanes served together read 16 different rows at one chunk index: XOR-ing the chunk
  // with (row / rows-per-256-bytes) puts them on 16 distinct 16-byte bank groups.
  __device__ static int f16(int r) { return (r / (256 / RB16)) & (C16 - 1); }
  __device__ static int f8(int r) { return (r / (256 / RB8)) & (C8 - 1); }
  // V rows are read by transposing 8-byte reads that touch 8 rows (keys 0-3 and 8-11 of a group of
  // 16) and 64 bytes of each: XOR-ing the chunk index of row r with fv(r) moves those 64-byte
  // pieces of rows r = 0..3 (mod 4) onto four different 64-byte bank groups.
  __device__ static int fv(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane T of the calling lane's 16-lane row (DPP row_newbcast; folds into the consuming VALU op).
template <int T>
__device__ __forceinline__ float row_bcast(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x150 + T, 0xF, 0xF, false));
}

__device__ __forceinline__ half2v pk(float a, float b) {
  return half2v{static_cast<_Float16>(a), static_cast<_Float16>(b)};  // v_cvt_pk_f16_f32 (RNE)
}

typedef __attribute__((address_space(3))) void lds_void;

// One direct global->LDS load per lane: 16 bytes from base + voff (base wave-uniform, in scalar
// registers; voff this lane's 32-bit byte offset) to lds_block + 16 * lane. The scalar-base form
// needs no per-load address arithmetic on the VALU. Written as inline assembly so that the
// compiler does not track it: every wait for it is explicit (dma_barrier), and the waits for LDS
// reads can count only the reads.
__device__ __forceinline__ void dma16(const char* base, uint32_t voff, char* lds_block) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds_block));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// The same with 4 bytes per lane, to lds_block + 4 * lane.
__device__ __forceinline__ void dma4(const char* base, uint32_t voff, char* lds_block) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)lds_block));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(base), "s"(lds) : "memory", "m0");
}

// Barrier after direct global->LDS loads. The memory fence of a workgroup barrier does not
// cover the LDS writes of these loads, so each wave first waits for all of its own outstanding
// loads (s_waitcnt with every counter at zero); after the barrier every wave's loads have landed.
__device__ __forceinline__ void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Row index inside a 32-key block that MFMA row r reads: bits 2 and 3 swapped.
__device__ __forceinline__ int perm32(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Direct global->LDS staging of the key-side tiles of one (sequence, KV head). Each wavefront
// loads fixed 1 KiB blocks of every tile; the per-lane source offsets of those blocks are
// computed once, so issuing a tile costs one address add per block.
template <int D, bool VN>
struct Stager {
  using L = Smem<D>;
  static constexpr int R16 = 1024 / L::RB16;  // K rows per 1 KiB block
  static constexpr int R8 = 1024 / L::RB8;
  static constexpr int NB16 = BN / R16;       // blocks per K tile
  static constexpr int NB8 = BN / R8;
  static constexpr int RV = 1024 / L::RBV;   // V rows per 1 KiB block
  static constexpr int NBV = BN / RV;
  static constexpr int I16 = (NB16 + NW - 1) / NW;  // blocks per wave
  static constexpr int I8 = (NB8 + NW - 1) / NW;
  static constexpr int IV = (NBV + NW - 1) / NW;

  // Uniform byte pointers (scalar registers) to the next tile of each stream, and per-lane byte
  // offsets of this wave's blocks inside a full tile (vector registers), so that a direct load is
  // one scalar-base + 32-bit-offset instruction and advancing a stream is one pointer add; only
  // the partial last tile of a sequence recomputes clamped rows. Each stream is consumed in tile
  // order, one call per tile.
  const char* k16;   // next K tile, fp16 rows
  const char* k8;    // next K tile, int8 rows
  const char* v;     // next V tile: fp16 rows (direct path) or the pre-pass's V^T tile
  const char* ks;    // k_scale of the next tile's first key
  int64_t st16;      // bytes between consecutive keys, fp16 K
  int64_t st8;       // bytes between consecutive keys, int8 K
  int64_t stv;       // bytes between consecutive keys, V
  uint32_t o16[I16], o8[I8], ov[IV];
  int w, Lk;
  int kn, vn, sn;    // index of the next K / V / factor tile
  int kfull;         // tiles [0, kfull) are whole

  __device__ void init(const FwdArgs& a, int k_begin, int hk, int Lk_, int w_, int64_t vt_tile0) {
    w = w_;
    Lk = Lk_;
    kn = vn = sn = 0;
    kfull = Lk / BN;
    st16 = a.k_stride_tok * 2;
    st8 = static_cast<int64_t>(a.hkv) * D;
    stv = a.v_stride_tok * 2;
    k16 = reinterpret_cast<const char*>(a.k) + k_begin * st16 + hk * a.k_stride_head * 2;
    k8 = reinterpret_cast<const char*>(a.k8) + static_cast<int64_t>(k_begin) * st8 + static_cast<int64_t>(hk) * D;
    v = VN ? reinterpret_cast<const char*>(a.v) + k_begin * stv + hk * a.v_stride_head * 2
           : reinterpret_cast<const char*>(a.vt + vt_tile0 * (D * BN));
    ks = reinterpret_cast<const char*>(a.k_scale + static_cast<int64_t>(hk) * a.total_k + k_begin);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < I16; ++i) o16[i] = off16(lane, i, BN);
#pragma unroll
    for (int i = 0; i < I8; ++i) o8[i] = off8(lane, i, BN);
#pragma unroll
    for (int i = 0; i < IV; ++i) ov[i] = VN ? offv(lane, i, BN) : static_cast<uint32_t>(lane * 16);
  }
  // byte offset of the chunk that lane loads in its i-th block of a tile whose rows past `last`
  // repeat row `last`
  __device__ uint32_t off16(int lane, int i, int last) const {
    const int row = (w + NW * i) * R16 + lane / L::C16;
    return static_cast<uint32_t>(min(row, last) * st16) + ((lane % L::C16) ^ L::f16(row)) * 16;
  }
  __device__ uint32_t off8(int lane, int i, int last) const {
    const int row = (w + NW * i) * R8 + lane / L::C8;
    return static_cast<uint32_t>(min(row, last) * st8) + ((lane % L::C8) ^ L::f8(row)) * 16;
  }
  __device__ uint32_t offv(int lane, int i, int last) const {
    const int row = (w + NW * i) * RV + lane / L::CV;
    return static_cast<uint32_t>(min(row, last) * stv) + ((lane % L::CV) ^ L::fv(row)) * 16;
  }

  // The next K tile into stage buf: fp16 rows if need16, int8 rows if need8. Rows past the
  // sequence end repeat the last key; the kernel masks them before use.
  __device__ __forceinline__ void k_next(char* buf, bool need16, bool need8) {
    __builtin_assume(w >= 0 && w < NW);
    const int lane = threadIdx.x & 63;
    if (__builtin_expect(kn < kfull, 1)) {
      if (need16) {
#pragma unroll
        for (int i = 0; i < I16; ++i)
          if (w + NW * i < NB16) dma16(k16, o16[i], buf + L::K16 + (w + NW * i) * 1024);
      }
      if (need8) {
#pragma unroll
        for (int i = 0; i < I8; ++i)
          if (w + NW * i < NB8) dma16(k8, o8[i], buf + L::K8 + (w + NW * i) * 1024);
      }
    } else {
      const int last = Lk - 1 - kn * BN;
      if (need16) {
#pragma unroll
        for (int i = 0; i < I16; ++i)
          if (w + NW * i < NB16) dma16(k16, off16(lane, i, last), buf + L::K16 + (w + NW * i) * 1024);
      }
      if (need8) {
#pragma unroll
        for (int i = 0; i < I8; ++i)
          if (w + NW * i < NB8) dma16(k8, off8(lane, i, last), buf + L::K8 + (w + NW * i) * 1024);
      }
    }
    k16 += BN * st16;
    k8 += BN * st8;
    ++kn;
  }

  // The next V tile into stage buf. Direct path: fp16 rows, those past the sequence end repeating
  // the last key (whose P is zero); V^T path: the pre-transposed tile, contiguous in the workspace.
  __device__ __forceinline__ void v_next(char* buf) {
    __builtin_assume(w >= 0 && w < NW);
    if constexpr (!VN) {
#pragma unroll
      for (int i = 0; i < IV; ++i)
        if (w + NW * i < NBV) dma16(v + (w + NW * i) * 1024, ov[i], buf + (w + NW * i) * 1024);
      v += D * BN * 2;
      return;
    }
    if (__builtin_expect(vn < kfull, 1)) {
#pragma unroll
      for (int i = 0; i < IV; ++i)
        if (w + NW * i < NBV) dma16(v, ov[i], buf + (w + NW * i) * 1024);
    } else {
      const int lane = threadIdx.x & 63;
      const int last = Lk - 1 - vn * BN;
#pragma unroll
      for (int i = 0; i < IV; ++i)
        if (w + NW * i < NBV) dma16(v, offv(lane, i, last), buf + (w + NW * i) * 1024);
    }
    v += BN * stv;
    ++vn;
  }

  // The k_scale of the next tile's 64 keys (keys past the sequence end repeat the last key's)
  // into a 256-byte factor slot: one 4-byte direct load per lane of the last wavefront.
  __device__ __forceinline__ void s_next(char* buf) {
    if (w == NW - 1) {
      const int lane = threadIdx.x & 63;
      const int key = sn < kfull ? lane : min(lane, Lk - 1 - sn * BN);
      dma4(ks, static_cast<uint32_t>(key * 4), buf);
    }
    ks += BN * 4;
    ++sn;
  }
};

typedef const __attribute__((address_space(4))) uint64_t const_u64;
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Workgroup-uniform metadata (sequence offsets, route words) is read through the constant
// address space, so that it lands in scalar registers via scalar loads; the kernel never writes it.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) { return ((const const_i32*)p)[i]; }

// Route bits of the workgroup's route rows for key-tile group gj: bit r = route row rr0 + r.
// The words are read through the constant address space (scalar loads); the kernel uses this for
// the first two tiles, before its loop.
__device__ __forceinline__ uint32_t group_bits(const const_u64* wrow, int wpr, int nrr, int gj) {
  uint32_t bits = 0;
  const int wi = gj >> 6, sh = gj & 63;
  for (int r = 0; r < nrr; ++r)
    bits |= static_cast<uint32_t>((wrow[static_cast<int64_t>(r) * wpr + wi] >> sh) & 1u) << r;
  return bits;
}

// Per-wavefront registers: constants of the wave's rows and the online-softmax state. KBLK: the K
// scales are constant over each 64-key tile (block-wise K quantization), so one factor per tile
// is folded into the per-row factor instead of multiplying every score.
template <int D, bool KV8, bool KBLK, bool VN>
struct Wave {
  int hl, my_q;
  int lim;         // last legal key (sequence-local) of this lane's query
  bool row_valid;
  uint64_t valid_lanes;  // wave-uniform ballot of row_valid
  // LDS byte offsets of this lane's operand rows: chunk (2*i + hl) ^ f of a row whose length is a
  // multiple of 128 bytes sits at row_start + 16*(hl ^ f) XOR 32*i, since 2*i + hl = 2*i ^ hl
  int kbase8, vbase;      // K8 row (i = ks), V^T row (i = 16-key step; V^T path)
  int vofs[D / 32];       // direct path: byte offset of this lane's transposing V read, per 32-channel block
  int kbase16;            // fp16 K row (i = ks)
  int fkey;               // key (within a 32-key half) whose factor this lane loads for its row
  int4v q8f[D / 32];
  half8v q16f[D / 16];  // fp16 Q fragments of this lane's query row: channels 16 ks + 8 hl + 0..7
  float cq;        // q_scale * softmax_scale * log2(e), floored so that 0 * -inf cannot occur
  float cs;        // softmax_scale * log2(e)
  float16v o[D / 32];  // O^T accumulator
  float16v s[2];       // fp32 scores of the two key halves, in units of 1 / c[half]
  float c[2];          // per-row factor of each half to log2 units: cq (INT8) or cs (FP16)
  half8v p[2][2][2];   // fp16 P of the two key halves of two tiles, [set][half][16-key step]
  float m, m_use, l;   // running max (log2 units), its finite stand-in, this lane's row sum
  bool have_max;       // wave-uniform: the first tile's slow path has run

  // s[0], s[1] = raw scores of the two key halves of the K tile in stage kst: int32
  // accumulators (as bits) for INT8, fp32 dot products for FP16; convert_f turns them into
  // scores. INT8: the eight K fragments are read first, then the two accumulator chains are
  // interleaved, so each MFMA waits only for its own fragment.
  __device__ __forceinline__ void qk_i8(const char* kst) {
    using L = Smem<D>;
    int4v kf[2][D / 32];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks)
        kf[kb][ks] = *reinterpret_cast<const int4v*>(kst + L::K8 + kb * 32 * L::RB8 + (kbase8 ^ (32 * ks)));
    int16v a0 = {}, a1 = {};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      a0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[0][ks], q8f[ks], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf[1][ks], q8f[ks], a1, 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 32), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * (D / 32), 0);
    s[0] = __builtin_bit_cast(float16v, a0);
    s[1] = __builtin_bit_cast(float16v, a1);
  }

  // FP16: the two chains interleaved, one Q fragment feeding both; the K fragments are read in
  // batches of four 16-channel steps (eight reads) ahead of their MFMAs, as in the INT8 route.
  __device__ __forceinline__ void qk_f16(const char* kst) {
    using L = Smem<D>;
    float16v a0 = {}, a1 = {};
#pragma unroll
    for (int bt = 0; bt < D / 64; ++bt) {
      half8v k0[4], k1[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ks = 4 * bt + j;
        k0[j] = *reinterpret_cast<const half8v*>(kst + L::K16 + (kbase16 ^ (32 * ks)));
        k1[j] = *reinterpret_cast<const half8v*>(kst + L::K16 + 32 * L::RB16 + (kbase16 ^ (32 * ks)));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0[j], q16f[4 * bt + j], a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1[j], q16f[4 * bt + j], a1, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    s[0] = a0;
    s[1] = a1;
  }

  // The V^T fragments of key half KB of the tile in stage vst (the A operand of the P.V MFMA:
  // lane l needs channel 32 dblk + l % 32 of keys 32 KB + 16 g8 + 8 (l / 32) + 0..7). V^T path:
  // one 16-byte read; direct path: two transposing reads of 4 keys each from the key-major rows.
  template <int KB>
  __device__ __forceinline__ void load_v(const char* vst, half8v (&vf)[2][D / 32]) const {
    if constexpr (!VN) {  // one 16-byte read per fragment from the V^T rows
#pragma unroll
      for (int g8 = 0; g8 < 2; ++g8)
#pragma unroll
        for (int dblk = 0; dblk < D / 32; ++dblk)
          vf[g8][dblk] = *reinterpret_cast<const half8v*>(vst + dblk * 32 * (BN * 2) + (vbase ^ (32 * (2 * KB + g8))));
      return;
    }
#pragma unroll
    for (int g8 = 0; g8 < 2; ++g8)
#pragma unroll
      for (int dblk = 0; dblk < D / 32; ++dblk) {
        const char* p = vst + vofs[dblk] + (32 * KB + 16 * g8) * (2 * D);
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)(p + 4 * (2 * D)));
        const int2v l2 = __builtin_bit_cast(int2v, lo), h2 = __builtin_bit_cast(int2v, hi);
        vf[g8][dblk] = __builtin_bit_cast(half8v, int4v{l2[0], l2[1], h2[0], h2[1]});
      }
  }

  // O^T += V^T P^T for key half KB from fragments already in registers.
  template <int KB, int SET>
  __device__ __forceinline__ void pv_regs(const half8v (&vf)[2][D / 32]) {
#pragma unroll
    for (int g8 = 0; g8 < 2; ++g8)
#pragma unroll
      for (int dblk = 0; dblk < D / 32; ++dblk)
        o[dblk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[g8][dblk], p[SET][KB][g8], o[dblk], 0, 0, 0);
  }

  // Debug dump of the raw INT8 accumulators of both halves (s holds them as bits): key j of
  // this lane's query row goes to dump_row[(j / bn_r) * tile_stride + j % bn_r], for the keys
  // j < Lk; key0 = sequence-local index of the tile's first key. Nothing when dump_row is NULL.
  __device__ __forceinline__ void dump_i8(int32_t* dump_row, int key0, int Lk, int bn_r, int tile_stride) const {
    if (dump_row == nullptr) return;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int key = key0 + 32 * kb + 16 * (t >> 3) + 8 * hl + (t & 7);
        const float v = s[kb][t];  // a plain value: bit_cast of a vector element reads element 0
        if (key < Lk) dump_row[(key / bn_r) * tile_stride + key % bn_r] = __builtin_bit_cast(int, v);
      }
  }

  // The per-key K scale of key half KB that this lane's 16-lane row broadcasts: lane i of a
  // row holds the factor of accumulator slot i of the row's lanes (key 16 (i / 8) + 8 hl + i % 8
  // of the half), so slot t reads it from lane t of its own row (DPP row_newbcast), and one
  // 4-byte LDS read per lane replaces the sixteen factors each lane would otherwise load.
  template <int KB>
  __device__ __forceinline__ float load_f(const float* scl) const {
    if constexpr (KBLK) return scl[0];  // the tile's one factor (that of its first key)
    return scl[32 * KB + fkey];
  }

  // Raw scores of half KB -> fp32 scores in units of 1 / c[KB], with the half's per-key factors
  // broadcast from fr. INT8: k_scale * (q8 . k8); FP16: the dot product (times k_scale for an INT8 cache).
  template <int KB, bool I8>
  __device__ __forceinline__ void convert_f(float fr) {
    if constexpr (KBLK) {
      // one factor for the whole tile: into the per-row factor (floored, as cq, so that a masked
      // -inf score never meets a zero factor)
      if constexpr (I8) {
#pragma unroll
        for (int t = 0; t < 16; ++t)
          s[KB][t] = static_cast<float>(__builtin_bit_cast(int, static_cast<float>(s[KB][t])));
        c[KB] = fmaxf(cq * fr, 1e-30f);
      } else {
        c[KB] = KV8 ? fmaxf(cs * fr, 1e-30f) : cs;
      }
    } else {
      if constexpr (I8 || KV8) convert_slots<KB, I8>(fr, std::make_integer_sequence<int, 16>{});
      c[KB] = I8 ? cq : cs;
    }
  }
  template <int KB, bool I8, int... T>
  __device__ __forceinline__ void convert_slots(float fr, std::integer_sequence<int, T...>) {
    ((s[KB][T] = (I8 ? static_cast<float>(__builtin_bit_cast(int, static_cast<float>(s[KB][T])))
                     : static_cast<float>(s[KB][T])) * row_bcast<T>(fr)), ...);
  }

  // Legality mask of half KB (causal diagonal, sequence tail): illegal scores become -inf.
  template <int KB>
  __device__ __forceinline__ void mask(int key0) {
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (key0 + 16 * (t >> 3) + 8 * hl + (t & 7) > lim) s[KB][t] = -INFINITY;
  }

  // p[KB] = fp16 exp2(s * c - m_use) of half KB; returns rs plus this lane's sum of the rounded
  // P (the second half continues the first half's sum).
  template <int KB, int SET>
  __device__ __forceinline__ float softmax(float rs) {
    const float ck = c[KB];
#pragma unroll
    for (int g8 = 0; g8 < 2; ++g8) {
      int4v pw;  // built from packed pairs, so that the slow path's join merges whole dwords
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float x0 = __builtin_fmaf(s[KB][8 * g8 + e], ck, -m_use);
        const float x1 = __builtin_fmaf(s[KB][8 * g8 + e + 1], ck, -m_use);
        const half2v h2 = pk(fast_exp2(x0), fast_exp2(x1));
        pw[e / 2] = __builtin_bit_cast(int, h2);
        rs = __builtin_amdgcn_fdot2(h2, half2v{static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)}, rs, false);
      }
      p[SET][KB][g8] = __builtin_bit_cast(half8v, pw);
    }
    return rs;
  }

  // The softmax of both halves of the current tile (P into set SET), with the P.V MFMAs of the
  // previous tile (P in set 1 - SET, V in stage vprev) among its instructions: the matrix core
  // works on the previous tile while the VALU exponentiates the current one. (Placing part of
  // the P.V inside the conversion, which is route-dependent code, made the compiler spill.)
  template <int SET>
  __device__ __forceinline__ float softmax_pv(const char* vprev) {
    half8v va[2][D / 32];
    load_v<0>(vprev, va);
    float rs = softmax<0, SET>(0.0f);
    pv_regs<0, 1 - SET>(va);
    half8v vb[2][D / 32];
    load_v<1>(vprev, vb);
    rs = softmax<1, SET>(rs);
    pv_regs<1, 1 - SET>(vb);
    return rs;
  }

  // Both halves of a tile after their softmax (P of each half against m_use): one slow-path
  // check for the tile; the slow path raises the max over both halves and recomputes both P.
  // EXACT (the FP16-state instance): the max is raised whenever a score exceeds it, as in the
  // plain online recurrence, so that P <= 1 and the row sum stays within binary16 range.
  template <bool EXACT, int SET>
  __device__ __forceinline__ void settle_tile(float rs) {
    float mx = -INFINITY;
    if constexpr (EXACT) {
#pragma unroll
      for (int t = 0; t < 16; ++t) mx = fmaxf(mx, fmaxf(s[0][t] * c[0], s[1][t] * c[1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mx = static_cast<float>(static_cast<_Float16>(mx));  // the max is state: binary16
    }
    // (lazy form: the first tile always takes the slow path, which gives every row with a legal
    // key its max; a row without one keeps m = -inf and P = 0)
    if ((EXACT || have_max)
            ? (__builtin_amdgcn_ballot_w64(EXACT ? mx > m : !(rs <= P_LIMIT)) & valid_lanes) != 0
            : true) {
      have_max = true;
      if constexpr (!EXACT) {
#pragma unroll
        for (int t = 0; t < 16; ++t) mx = fmaxf(mx, fmaxf(s[0][t] * c[0], s[1][t] * c[1]));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
      }
      if (mx > m) {
        const float alpha = fast_exp2(m - mx);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
        l *= alpha;
        m = mx;
        m_use = mx;
      }
      rs = softmax<1, SET>(softmax<0, SET>(0.0f));
    }
    l += rs;
  }

  // The state kept between tiles rounded to binary16 (round to nearest even) and widened back:
  // this lane's part of the row sum and O (the running max is rounded where it is raised, before
  // P and the rescale factor are computed from it).
  __device__ __forceinline__ void round_state_fp16() {
    l = static_cast<float>(static_cast<_Float16>(l));
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int t = 0; t < 16; ++t) o[i][t] = static_cast<float>(static_cast<_Float16>(o[i][t]));
  }
};

// Where the debug dump of the current tiles goes (DUMP instances only).
struct DumpCtx {
  int32_t* row;  // this lane's query row in the dump (NULL: not dumped); see Wave::dump_i8
  int bn_r, tile_stride, Lk;
  int act_limit;  // a key tile starting at j0 is dumped iff j0 <= act_limit
};

// Fused Q quantization (the alternative to the quantize-once pass): the two lanes of a query row
// (hl = 0, 1) hold its fp16 channels 16 k + 8 hl + 0..7 (k = 0 .. D/16-1); they share the row's
// absolute maximum and compute the same codes and scale as the quantize-once pass (same fp32
// operations: a = max|x|, inv = 127 / a and a / 127 correctly rounded, rint, clamp). The INT8
// score MFMA wants lane hl to hold channels 32 ks + 16 hl + 0..15, so each lane then swaps one
// 8-code group per 32 channels with its partner lane (lane ^ 32). Returns the scale. Every lane
// of the wavefront must call it (the exchanges are wave-wide).
template <int D>
__device__ __forceinline__ float quantize_q_regs(const half8v (&q16f)[D / 16], int hl, int4v (&q8f)[D / 32]) {
  float am = 0.0f;
#pragma unroll
  for (int k = 0; k < D / 16; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(static_cast<float>(q16f[k][e])));
  am = fmaxf(am, __shfl_xor(am, 32));  // the row's other half
  float s = 0.0f;
  float inv = 0.0f;
  if (am > 0.0f) {
    inv = 127.0f / am;
    s = am / 127.0f;
  }
  int2v codes[D / 16];  // 8 codes of each fp16 fragment
#pragma unroll
  for (int k = 0; k < D / 16; ++k) {
    int2v packed = {};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c = rintf(static_cast<float>(q16f[k][e]) * inv);
      c = fminf(fmaxf(c, -127.0f), 127.0f);
      packed[e / 4] |= static_cast<int>(static_cast<uint32_t>(static_cast<uint8_t>(static_cast<int8_t>(c))) << (8 * (e % 4)));
    }
    codes[k] = packed;
  }
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    // lane hl = 0 keeps channels 32 ks + 0..7 and needs 32 ks + 8..15 (the partner's fragment
    // 2 ks); lane hl = 1 keeps 32 ks + 24..31 and needs 32 ks + 16..23 (the partner's 2 ks + 1)
    const int2v send = hl ? codes[2 * ks] : codes[2 * ks + 1];
    int2v recv;
    recv[0] = __shfl_xor(send[0], 32);
    recv[1] = __shfl_xor(send[1], 32);
    const int2v lo = hl ? recv : codes[2 * ks];
    const int2v hi = hl ? codes[2 * ks + 1] : recv;
    q8f[ks] = int4v{lo[0], lo[1], hi[0], hi[1]};
  }
  return s;
}

// Instances of the fused kernel. Production streams tile n+1 into the second stage while tile n
// is computed. The others are debug and numerics instances:
//   kDump  writes the raw INT8 accumulators of every computed INT8-routed tile;
//   kKblk  takes one K scale per 64-key tile (block-wise K scales);
//   kSync  single-buffered: loads tile n into the one stage, waits, then computes it; its
//          results must equal the production instance's bit for bit (a staging race would show
//          as a difference);
//   kF16s  rounds the online-softmax state (m, l and O) to binary16 after every 64-key tile.
enum Variant : int { kProd = 0, kDump = 1, kKblk = 2, kSync = 3, kF16s = 4 };

// One work item: the workgroup-sized piece (bx, by, bz) of the grid (query heads, query tiles in
// reverse order, sequences) that a one-workgroup-per-item launch would give blockIdx.
template <int D, bool KV8, int VAR, bool VN>
__device__ __forceinline__ void prefill_item(const FwdArgs& a, char* smem, int bx, int by, int bz) {
  constexpr bool DUMP = VAR == kDump;
  constexpr bool KBLK = VAR == kKblk;
  constexpr bool SYNC = VAR == kSync;
  constexpr bool F16S = VAR == kF16s;
  using L = Smem<D>;

  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));  // per item: nothing lane-dependent is kept live across items
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform (scalar)
  const int hl = lane >> 5;   // half of the wave: selects 8 of the 16 keys of a k-step
  const int r32 = lane & 31;  // query row of this lane within the wave

  // XCD-friendly head order: consecutive workgroups cycle through the KV heads first
  const int x = bx;
  const int grp = a.hq / a.hkv;
  const int b = bz;
  const int n_ct = (a.max_seqlen_q + BM - 1) / BM;
  int h, c;
  if (a.hkv % 8 == 0 && n_ct >= 64) {
    // long sequences, KV heads a multiple of 8: workgroup lin of a sequence runs on XCD lin % 8,
    // which takes its KV heads j, j + 8, ... one at a time: the k-th workgroup it receives is
    // query tile c (heaviest first) of query head r % grp of its KV head k / (grp n_ct)
    const int lin = x + a.hq * by;
    const int j = lin & 7, k = lin >> 3;
    const int per_kv = grp * n_ct;
    const int r = k % per_kv;
    c = n_ct - 1 - r / grp;
    h = (j + 8 * (k / per_kv)) * grp + r % grp;
  } else {
    h = grp * (x % a.hkv) + x / a.hkv;
    c = n_ct - 1 - by;
  }
  const int q_begin = ld_uniform(a.cu_q, b);
  const int Lq = ld_uniform(a.cu_q, b + 1) - q_begin;
  const int k_begin = ld_uniform(a.cu_k, b);
  const int Lk = ld_uniform(a.cu_k, b + 1) - k_begin;
  const int q0 = c * BM;
  if (q0 >= Lq) return;  // uniform over the workgroup

  const int hk = h / grp;
  const int off = Lk - Lq;  // bottom-right causal alignment
  const int q_last = min(q0 + BM, Lq) - 1;
  const int key_end = a.causal ? min(Lk, q_last + off + 1) : Lk;
  const int n_tiles = key_end > 0 ? (key_end + BN - 1) / BN : 0;

  const int qa = q0 + ROWS_W * w;  // first query row of this wave
  const bool wave_live = qa < Lq;
  const int qlast_w = min(qa + ROWS_W - 1, Lq - 1);
  // tiles [0, n_full) need no legality mask for any row of this wave; tiles [n_wave, n_tiles)
  // hold no legal key for any of its rows (the far side of the workgroup's causal diagonal
  // block). The wave computes tile n_wave (all its scores masked, P = 0), whose iteration runs
  // the P.V of its last real tile, and skips the tiles after it: they would add exact zeros.
  const int n_full = (a.causal ? min(Lk, qa + off + 1) : Lk) / BN;
  const int n_wave = !wave_live ? -1 : a.causal ? (max(0, min(Lk, qlast_w + off + 1)) + BN - 1) / BN : n_tiles;

  // route rows of the workgroup and the wave's own one
  const int mt0 = ld_uniform(a.cu_mtiles, b);
  const int rr0 = q0 / a.bm_r;
  const int nrr = q_last / a.bm_r - rr0 + 1;
  const int my_rl = wave_live ? qa / a.bm_r - rr0 : 0;
  const uint32_t full = (1u << nrr) - 1u;
  const const_u64* wrow = (const const_u64*)(a.words) +  // scalar loads; the words are read-only here
                          (static_cast<int64_t>(hk) * a.total_mtiles + mt0 + rr0) * a.wpr;
  const int tpg = (a.bn_r / BN) * a.group;  // pipeline tiles per routing bit

  Stager<D, VN> stg;
  int tiles_before = 0;  // V^T path: 64-key tiles of the sequences before b (tiles never straddle sequences)
  if (!VN)
    for (int i = 0; i < b; ++i) tiles_before += (ld_uniform(a.cu_k, i + 1) - ld_uniform(a.cu_k, i) + BN - 1) / BN;
  stg.init(a, k_begin, hk, Lk, w, static_cast<int64_t>(hk) * a.vt_tiles + tiles_before);
  char* const kbuf = smem + L::KBUF;
  char* const vbuf = smem + L::VBUF;
  char* const sbuf = smem + L::SBUF;

  Wave<D, KV8, KBLK, VN> wv;
  wv.hl = hl;
  wv.my_q = qa + r32;
  wv.lim = a.causal ? min(Lk - 1, wv.my_q + off) : Lk - 1;
  wv.row_valid = wv.my_q < Lq;
  wv.valid_lanes = __builtin_amdgcn_ballot_w64(wv.row_valid);
  {
    const int kr = perm32(r32);  // K row this lane feeds to the MFMA
    wv.kbase16 = kr * L::RB16 + 16 * (hl ^ L::f16(kr));
    wv.kbase8 = kr * L::RB8 + 16 * (hl ^ L::f8(kr));
    wv.vbase = r32 * (BN * 2) + 16 * (hl ^ vt_swizzle(r32));
    // transposing V reads: lane m of 16-lane group g supplies key row 8 (g >> 1) + (m >> 2) and
    // channels 16 (g & 1) + 4 (m & 3) .. + 3, and receives channel 16 (g & 1) + m of 4 keys
    const int g = lane >> 4, m = lane & 15;
    const int vrow = 8 * (g >> 1) + (m >> 2);
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk) {
      const int chunk = 4 * dblk + 2 * (g & 1) + ((m & 3) >> 1);  // 16-byte chunk of the channels
      wv.vofs[dblk] = vrow * L::RBV + (chunk ^ L::fv(vrow)) * 16 + 8 * (m & 1);
    }
    wv.fkey = 16 * ((lane & 15) >> 3) + 8 * hl + (lane & 7);
  }

  // ---- resident queries, in registers: each lane's fp16 Q fragments (the B operand of the FP16
  // score MFMAs) straight from global memory, and its int8 Q fragments
  if (wv.row_valid) {
    const _Float16* qrow = a.q + (q_begin + wv.my_q) * a.q_stride_tok + static_cast<int64_t>(h) * a.q_stride_head;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) wv.q16f[ks] = *reinterpret_cast<const half8v*>(qrow + 16 * ks + 8 * hl);
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) wv.q16f[ks] = half8v{};
  }
  wv.cq = 1e-30f;
  wv.cs = a.scale_log2;
  if (wv.row_valid && a.q8 != nullptr) {  // quantize-once: codes and scale from the a1 pass
    const int64_t tq = q_begin + wv.my_q;
    const int8_t* q8p = a.q8 + (tq * a.hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) wv.q8f[ks] = *reinterpret_cast<const int4v*>(q8p + 32 * ks + 16 * hl);
    wv.cq = fmaxf(a.q_scale[static_cast<int64_t>(h) * a.total_q + tq] * a.scale_log2, 1e-30f);
  } else {  // rows past the sequence; with fused quantization the codes are set further down
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) wv.q8f[ks] = int4v{};
  }
#pragma unroll
  for (int i = 0; i < D / 32; ++i) wv.o[i] = float16v{};
  wv.m = -INFINITY;
  wv.have_max = false;
  wv.m_use = 0.0f;
  wv.l = 0.0f;

  DumpCtx dc{};
  if (DUMP) {
    const int my_rr = mt0 + qa / a.bm_r;
    const bool dump_me = h == a.dump_head && wave_live && wv.row_valid && my_rr >= a.dump_m0 &&
                         my_rr < a.dump_m0 + a.dump_mcount;
    dc.row = dump_me ? a.dump + (static_cast<int64_t>(my_rr - a.dump_m0) * a.dump_ntiles * a.bm_r +
                                 wv.my_q % a.bm_r) * a.bn_r
                     : nullptr;
    dc.bn_r = a.bn_r;
    dc.tile_stride = a.bm_r * a.bn_r;
    dc.Lk = Lk;
    dc.act_limit = a.causal ? qlast_w + off : 0x7fffffff;
  }

  // route bits of the workgroup's rows for tiles n and n+1 (bit r = route row rr0 + r)
  auto bits_of = [&](int n) { return group_bits(wrow, a.wpr, nrr, n / tpg); };
  uint32_t rb0 = n_tiles > 0 ? bits_of(0) : 0u;
  uint32_t rb1 = n_tiles > 1 ? bits_of(1) : 0u;
  int pos2 = 2 % tpg, grp2 = 2 / tpg;  // routing group of tile 2 and the tile's place in it

  // fused Q quantization: each lane quantizes its half of its query row from its fp16 fragments
  if (a.q8 == nullptr) {
    const float qs = quantize_q_regs<D>(wv.q16f, hl, wv.q8f);  // every lane: exchanges with lane ^ 32
    if (wv.row_valid) wv.cq = fmaxf(qs * a.scale_log2, 1e-30f);
  }

  // ---- prologue: K, V and factors of tile 0 (the single-buffered instance loads every tile in
  // its own iteration)
  if (!SYNC && n_tiles > 0) {
    stg.k_next(kbuf, rb0 != full, rb0 != 0u);
    stg.v_next(vbuf);
    stg.s_next(sbuf);
  }

  // ---- main loop. Iteration n: the direct loads of tile n+1 fly while tile n is computed. Each
  // wavefront issues the score MFMAs of tile n, converts them, and runs the softmax of tile n with
  // the P.V MFMAs of tile n-1 among its VALU instructions, so its own matrix-core work overlaps
  // its exponentials. P alternates between two register sets (the loop is unrolled by two); V
  // keeps three stages (tiles n-1, n, n+1), K and the factors two. Iteration 0's "tile -1" is a
  // zeroed V stage times zero P, which adds exact zeros to O. The single-buffered instance loads
  // K, V and the factors of tile n in its own iteration and waits for them.
  int vs_prev = 2, vs_cur = 0, vs_next = 1;  // V stages of tiles n-1, n, n+1
#pragma unroll
  for (int i = tid * 16; i < L::VSTAGE; i += NW * 64 * 16)
    *reinterpret_cast<int4v*>(vbuf + vs_prev * L::VSTAGE + i) = int4v{};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int g8 = 0; g8 < 2; ++g8) wv.p[1][kb][g8] = half8v{};
  // Route words of later routing groups: lane r < nrr loads route row r's word with a vector load
  // at the top of the iteration before the group starts, and a ballot of the bits forms the
  // group's route bits at the end of it, so no scalar-load wait sits in the loop.
  const uint64_t* wrow_v = reinterpret_cast<const uint64_t*>(a.words) +
                           (static_cast<int64_t>(hk) * a.total_mtiles + mt0 + rr0 + min(lane, nrr - 1)) * a.wpr;
  uint64_t word2 = 0;
  auto iter = [&](auto set_c, int n) {
    constexpr int SET = decltype(set_c)::value;
    dma_barrier();  // tile n landed; the K / factor stages of tile n-1 and the V stage of n-2 are free
    const bool fetch = pos2 == 0 && n + 2 < n_tiles;  // tile n+2 starts a routing group (uniform)
    if (fetch) word2 = wrow_v[grp2 >> 6];
    if constexpr (SYNC) {
      stg.k_next(kbuf, rb0 != full, rb0 != 0u);
      stg.v_next(vbuf + vs_cur * L::VSTAGE);
      stg.s_next(sbuf);
      dma_barrier();
    } else if (n + 1 < n_tiles) {
      stg.k_next(kbuf + ((n + 1) & 1) * L::KSTAGE, rb1 != full, rb1 != 0u);
      stg.v_next(vbuf + vs_next * L::VSTAGE);
      stg.s_next(sbuf + ((n + 1) & 1) * L::SSLOT);
    }
    if (n <= n_wave) {
      const int j0 = n * BN;
      const bool i8 = (rb0 >> my_rl) & 1u;
      const int st = SYNC ? 0 : (n & 1);
      const char* kst = kbuf + st * L::KSTAGE;
      const float* scl = reinterpret_cast<const float*>(sbuf + st * L::SSLOT);
      if (i8) {
        wv.qk_i8(kst);
        if constexpr (DUMP) wv.dump_i8(j0 <= dc.act_limit ? dc.row : nullptr, j0, dc.Lk, dc.bn_r, dc.tile_stride);
      } else {
        wv.qk_f16(kst);
      }
      const float f0 = wv.template load_f<0>(scl);
      const float f1 = wv.template load_f<1>(scl);
      if (i8) {
        wv.template convert_f<0, true>(f0);
        wv.template convert_f<1, true>(f1);
      } else {
        wv.template convert_f<0, false>(f0);
        wv.template convert_f<1, false>(f1);
      }
      if (n >= n_full) {
        wv.template mask<0>(j0);
        wv.template mask<1>(j0 + 32);
      }
      const float rs = wv.template softmax_pv<SET>(vbuf + vs_prev * L::VSTAGE);
      if constexpr (F16S) wv.round_state_fp16();  // the state after tile n-1
      wv.template settle_tile<F16S, SET>(rs);
    }
    const int vs_free = vs_prev;
    vs_prev = vs_cur;
    vs_cur = vs_next;
    vs_next = vs_free;
    rb0 = rb1;
    // tile n+2's position in its routing group, kept as a counter (no division per tile)
    if (fetch)
      rb1 = static_cast<uint32_t>(__builtin_amdgcn_ballot_w64(lane < nrr && ((word2 >> (grp2 & 63)) & 1u) != 0u));
    if (++pos2 == tpg) {
      pos2 = 0;
      ++grp2;
    }
  };
  for (int n = 0; n < n_tiles; n += 2) {
    iter(std::integral_constant<int, 0>{}, n);
    if (n + 1 == n_tiles) break;
    iter(std::integral_constant<int, 1>{}, n + 1);
  }
  if (n_wave == n_tiles && n_tiles > 0) {  // P.V of the last tile, whose P is in set (n_tiles - 1) & 1
    const char* vst = vbuf + vs_prev * L::VSTAGE;
    half8v va[2][D / 32], vb[2][D / 32];
    wv.template load_v<0>(vst, va);
    wv.template load_v<1>(vst, vb);
    if ((n_tiles - 1) & 1) {
      wv.template pv_regs<0, 1>(va);
      wv.template pv_regs<1, 1>(vb);
    } else {
      wv.template pv_regs<0, 0>(va);
      wv.template pv_regs<1, 0>(vb);
    }
    if constexpr (F16S) wv.round_state_fp16();
  }

  // ---- epilogue: O = O^T / l, LSE = (m + log2 l) * ln 2
  const float l_row = wv.l + __shfl_xor(wv.l, 32);
  if (!wv.row_valid) return;
  const int64_t tq = q_begin + wv.my_q;
  const float inv_l = l_row > 0.0f ? 1.0f / l_row : 0.0f;
  if (a.out_f32) {
    float* op = static_cast<float*>(a.out) + (tq * a.hq + h) * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float4v v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = wv.o[dblk][4 * g4 + e] * inv_l;
        *reinterpret_cast<float4v*>(op + dblk * 32 + 8 * g4 + 4 * hl) = v4;
      }
  } else {
    _Float16* op = static_cast<_Float16*>(a.out) + (tq * a.hq + h) * D;
#pragma unroll
    for (int dblk = 0; dblk < D / 32; ++dblk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        half4v v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = static_cast<_Float16>(wv.o[dblk][4 * g4 + e] * inv_l);
        *reinterpret_cast<half4v*>(op + dblk * 32 + 8 * g4 + 4 * hl) = v4;
      }
  }
  if (a.lse != nullptr && hl == 0)
    a.lse[static_cast<int64_t>(h) * a.total_q + tq] =
        l_row > 0.0f ? (wv.m_use + log2f(l_row)) * 0.69314718055994531f : -INFINITY;
}


// The fused kernel. PERS = false: one workgroup per work item (grid = items). PERS = true
// (persistent, V^T path): as many workgroups as fit on the device at once, each taking items from
// eight queues in the workspace, queue i holding the items g = i (mod 8) of the linear item order
// g = x + hq (y + n_ct z) in increasing order -- the items the hardware would deal to XCD i. A
// workgroup serves its own XCD's queue (the XCC id register) first and then the others, so an XCD
// that runs faster than the rest takes over their last (lightest) items instead of idling: the
// XCDs of one device do not run equally fast. Every workgroup leaves once all queues are empty.
template <int D, bool KV8, int VAR, bool VN, bool PERS>
__global__ __launch_bounds__(NW * 64, 1) void prefill_fwd_kernel(const FwdArgs a, int n_items) {
  using L = Smem<D>;
  __shared__ __attribute__((aligned(1024))) char smem[L::BYTES];
  if constexpr (!PERS) {
    prefill_item<D, KV8, VAR, VN>(a, smem, blockIdx.x, blockIdx.y, blockIdx.z);
  } else {
    __shared__ int item_sh;
    const int n_ct = (a.max_seqlen_q + BM - 1) / BM;
    const int xq = static_cast<int>(__builtin_amdgcn_s_getreg(20 | (0 << 6) | (31 << 11)) & 7);  // XCC id
    for (;;) {
      if (threadIdx.x == 0) {
        int g = -1;
        for (int i = 0; i < 8 && g < 0; ++i) {
          const int qi = (xq + i) & 7;
          const int nq = qi < n_items ? (n_items - qi + 7) / 8 : 0;
          if (nq == 0) continue;
          const int k = atomicAdd(&a.sched[qi], 1);  // vector atomic; counters only grow
          if (k < nq) g = qi + 8 * k;
        }
        item_sh = g;
      }
      __syncthreads();
      const int g = item_sh;
      __syncthreads();  // item_sh is rewritten only after every wave has read it
      if (g < 0) break;
      prefill_item<D, KV8, VAR, VN>(a, smem, g % a.hq, (g / a.hq) % n_ct, g / (a.hq * n_ct));
    }
  }
}

// Workgroups of one instance resident on the current device at once (cached per device).
template <typename K>
int resident_workgroups(K kern) {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n_cu = 0, occ = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, reinterpret_cast<const void*>(kern), NW * 64, 0) != hipSuccess)
      return 0;
    cache[dev] = n_cu * (occ > 0 ? occ : 1);
  }
  return cache[dev];
}

template <int D, bool KV8, int VAR, bool VN>
hipError_t launch_i(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  const int n_items = static_cast<int>(grid.x * grid.y * grid.z);
  if constexpr (!VN) {
    if (a.sched != nullptr) {
      const int n_res = resident_workgroups(prefill_fwd_kernel<D, KV8, VAR, VN, true>);
      if (n_res > 0) {
        prefill_fwd_kernel<D, KV8, VAR, VN, true><<<dim3(n_items < n_res ? n_items : n_res), dim3(NW * 64), 0, stream>>>(a, n_items);
        return hipGetLastError();
      }
    }
  }
  prefill_fwd_kernel<D, KV8, VAR, VN, false><<<grid, dim3(NW * 64), 0, stream>>>(a, n_items);
  return hipGetLastError();
}

template <int D, bool KV8, bool VN>
hipError_t launch_v(const FwdArgs& a, dim3 grid, hipStream_t stream) {
  // the debug dump of the INT8 accumulators is compiled into a separate instance of the kernel
  // (with the dump the per-key instance runs: block-wise scales are per-key scales too)
  if (a.dump != nullptr) return launch_i<D, KV8, kDump, VN>(a, grid, stream);
  if (a.sync_stages) return launch_i<D, KV8, kSync, VN>(a, grid, stream);
  if (a.state_fp16) return launch_i<D, KV8, kF16s, VN>(a, grid, stream);
  if (a.k_block > 0) return launch_i<D, KV8, kKblk, VN>(a, grid, stream);
  return launch_i<D, KV8, kProd, VN>(a, grid, stream);
}

template <int D, bool KV8>
hipError_t launch_t(const FwdArgs& a, int32_t batch, hipStream_t stream) {
  const int n_ct = (a.max_seqlen_q + BM - 1) / BM;
  if (n_ct == 0 || batch == 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.hq), static_cast<unsigned>(n_ct), static_cast<unsigned>(batch));
  return a.v_direct ? launch_v<D, KV8, true>(a, grid, stream) : launch_v<D, KV8, false>(a, grid, stream);
}

}  // namespace

hipError_t launch_prefill(const FwdArgs& a, int32_t batch, int32_t head_dim, bool kv_int8,
                          hipStream_t stream) {
  if (head_dim == 128)
    return kv_int8 ? launch_t<128, true>(a, batch, stream) : launch_t<128, false>(a, batch, stream);
  return kv_int8 ? launch_t<64, true>(a, batch, stream) : launch_t<64, false>(a, batch, stream);
}

}  // namespace tilemix
