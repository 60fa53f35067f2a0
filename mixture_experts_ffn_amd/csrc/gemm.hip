// Grouped GEMMs of the MoE FFN block on gfx950 bf16 MFMA, fp32 accumulation.
//
// Two epilogues share one tiled main loop (C = A * B^T, both operands
// K-contiguous):
//   gate/up  (Inferentia2 bf16 card, "How it works (the recipe)": the fused
//            gate_up linear): each wavefront holds 16 gate columns and the 16
//            matching up columns, so the epilogue forms gelu_tanh(gate) * up in
//            registers and writes the bf16 intermediate h.
//   down     (the down linear): the epilogue multiplies each grouped row by its
//            router weight (if any) and writes bf16 rows, or writes fp32.
// A rows may be gathered (the tokens of an expert, in grouped order), so the
// routed pairs are computed without copying x. int8 weights (int8 experts card,
// "How it works") are widened to bf16 exactly in registers and their per-row
// fp32 scales are applied in the epilogue. E4M3 weights (the vLLM recipe's fp8
// variant) meet A rows quantised per token to E4M3 bytes in gfx950's fp8 MFMA
// (16x16x128, twice the bf16 rate: a K-step there is 128 codes, 128 bytes a
// row, the bytes a bf16 K-step of 64 moves), both scales applied per row and
// column in the epilogue. The template parameter WQ names the format: 0 bf16,
// 1 int8, 2 E4M3. combine_kernel then adds, per token,
// the dense output and its K weighted expert rows (ONNX export card, "Truthful
// graph contracts", row "MoE topology": dense + moe).
//
// Tile 256 x 256 x 64, 512 threads = 8 wavefronts side by side in N, each
// owning all 256 rows and 32 columns (16 x 2 MFMA 16x16x32 tiles); 16-row slabs
// past the tile's last valid row (in groups of four) skip their MFMAs. With
// about 128 routed rows per expert a 256-row tile holds an expert's rows in one
// M-tile, so each weight tile streams through a CU once per expert.
//
// The weights (B) are the stream that HBM bounds. They are stored tiled (16
// rows x 64 k per tile, in the order of the MFMA operand: lane l holds column
// l % 16, k 16 (l / 16) .. + 16), so each wavefront loads its own B fragments
// straight from global memory into registers as contiguous 1 KB runs, through
// a ring of kDepth K-steps, without passing through LDS. The activations (A,
// shared by all wavefronts) move from global memory straight into LDS
// (global_load_lds_dwordx4: each lane's 16 bytes land at the wavefront's LDS
// base + 16 * lane, so the lanes fetch the XOR-swizzled chunk order directly)
// through kDepth LDS stages, which the epilogue reuses to stage its output.
// Both run kDepth - 1 K-steps ahead: about 192 KB per CU in flight. Blocks
// are mapped XCD-aware (gemm_expert_blocks): block b runs on XCD b % 8, and
// each XCD owns a contiguous run of M-tiles with all their N-tiles, so an
// M-tile's A rows and an expert's weight tiles meet in the same L2. A launch
// carries two problems (the routed experts and the dense MLP) back to back.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = 64;
constexpr int kHalfN = BN / 2;  // gate/up: h columns per tile
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = kGemmXcds;
constexpr int kDepth = 4;       // K-steps in flight per wavefront: A stages and B slots
constexpr int kSlabs = BM / 16;
constexpr int kADma = BM / kWaves / 8;  // A loads (8 rows, 1 KB each) per wavefront per K-step
enum { MODE_GATEUP = 0, MODE_DOWN = 1 };
static_assert(BM == 256 && kWaves * 32 == BN, "8 wavefronts x 32 columns, 256 rows");

// LDS position of A's 16-byte chunk c (of 8) of tile row r: chunk c ^ f(r),
// f(r) = (r & 7) ^ ((r >> 3) & 1). A 128-bit LDS read serves 16 lanes a cycle
// across 64 banks (256 B, two 128-byte rows' worth): the MFMA A fragments read
// chunk c of rows R .. R + 15 (R a multiple of 16), which must land on 16
// distinct (row parity, chunk) bank groups, and f gives that (r & 7 alone maps
// rows r and r + 8 onto the same banks: a two-way conflict on every fragment
// read). f depends on r % 16 only, so a wavefront's fragment addresses differ
// between slabs by a constant offset.
__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ a_swz(r)) << 3); }

template <int MODE>
__host__ __device__ __forceinline__ int n_tiles_of(const GemmArgs& p) {
    return MODE == MODE_GATEUP ? (p.n_out + kHalfN - 1) / kHalfN : p.n_out / BN;
}
__host__ __device__ __forceinline__ int mtile_cap(const GemmArgs& p) {
    return p.mtile_group ? p.max_mtiles : (p.M_dense + BM - 1) / BM;
}
// The dense problem's M-tiles are cut into gm groups (gm | kXcds). Its units
// (M-tile, N-tile) are ordered by group, then N-tile, then M-tile, and each XCD
// runs one contiguous, equal share of them, about kXcdSlots at a time: such a
// pass reads each of its M-tiles' rows and N-tiles' weights (tiles of equal
// size, BM = BN) from HBM once, the other blocks of the pass finding them in
// the XCD's L2. gm minimises the tiles the passes read: at T = 2048 (8 M-tiles)
// 4 M-tiles x 4-5 N-tiles per XCD instead of 1 x 17 (weights read 8 times).
constexpr int kXcdSlots = 32;  // blocks in flight per XCD: 32 CUs, one block each
template <int MODE>
__host__ __device__ __forceinline__ int dense_groups(const GemmArgs& p) {
    const int m_total = (p.M_dense + BM - 1) / BM;
    const int share = (m_total * n_tiles_of<MODE>(p) + kXcds - 1) / kXcds;
    const int pass = min(share, kXcdSlots), passes = (share + pass - 1) / pass;
    int best = 1, best_cost = 0;
    for (int g = 1; g <= kXcds; g *= 2) {
        const int m_in = (m_total + g - 1) / g, pm = min(m_in, pass);
        const int cost = passes * (pm + (pass + pm - 1) / pm);
        if (g == 1 || cost < best_cost) {
            best = g;
            best_cost = cost;
        }
    }
    return best;
}
template <int MODE>
__host__ __device__ __forceinline__ int blocks_of(const GemmArgs& p) {
    if (p.mtile_group) return kXcds * ((p.max_mtiles + kXcds - 1) / kXcds) * n_tiles_of<MODE>(p);
    const int units = ((p.M_dense + BM - 1) / BM) * n_tiles_of<MODE>(p);
    return kXcds * ((units + kXcds - 1) / kXcds);
}

// tiled-layout tile (16 weight rows) holding the wavefront's column tile j
// (gate/up: tile 0 holds gate rows, tile 1 the matching up rows; h columns
// past the end repeat the last tile, and their results are never stored)
template <int MODE>
__device__ __forceinline__ int b_tile(const GemmArgs& p, int nt, int wn, int j) {
    if (MODE == MODE_GATEUP) {
        const int ht = min(nt * (kHalfN / 16) + wn, p.n_out / 16 - 1);
        return j == 0 ? ht : p.up_off / 16 + ht;
    }
    return (nt * BN + wn * 32 + j * 16) / 16;
}

// two int8 of a word (bytes sh, sh+1) -> two bf16 (exact: |q| <= 127 fits the bf16 significand)
__device__ __forceinline__ unsigned i8pair_to_bf16(unsigned word, int sh) {
    const float a = (float)(int8_t)((word >> sh) & 0xFF);
    const float b = (float)(int8_t)((word >> (sh + 8)) & 0xFF);
    return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
// native 4 x u32 vector (a first-class type that stays in registers)
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

constexpr int kAStageElems = BM * BK;  // bf16 elements per LDS stage of A

// One K-step of the wavefront's B fragments: bf16 q[2 j + s] = column tile j,
// 8 k of sub-step s; int8 q[j] = column tile j, all 16 k; E4M3 q[2 j + s] =
// column tile j, the 16 codes of 64-wide tile s of the 128-wide K-step.
template <int WQ>
struct BStep {
    v4u q[WQ == 1 ? 2 : 4];
};
template <int WQ>
constexpr int kBLoads = WQ == 1 ? 2 : 4;
typedef int v8i __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v8i cat8(const v4u& a, const v4u& b) {
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

// bp[j]: this lane's 16-byte piece of tile 0 of the wavefront's tile row j; a
// tile is 2 KB bf16 (sub-step s at + 1024 s) or 1 KB int8 or E4M3, so every
// load of the wavefront reads one contiguous 1 KB. A K-step is one tile (bf16,
// int8) or two (E4M3: tiles 2 kt and 2 kt + 1; the second repeats the first
// past the last tile of an odd count, where the A codes are zero).
template <int WQ>
__device__ __forceinline__ void b_load(const char* const (&bp)[2], int kt, int nkt, BStep<WQ>& r) {
    if (WQ == 2) {
        const int64_t o0 = (int64_t)(2 * kt) * 1024, o1 = (int64_t)min(2 * kt + 1, nkt - 1) * 1024;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            r.q[2 * j] = *reinterpret_cast<const v4u*>(bp[j] + o0);
            r.q[2 * j + 1] = *reinterpret_cast<const v4u*>(bp[j] + o1);
        }
    } else if (WQ == 1) {
        const int64_t off = (int64_t)kt * 1024;
#pragma unroll
        for (int j = 0; j < 2; ++j) r.q[j] = *reinterpret_cast<const v4u*>(bp[j] + off);
    } else {
        const int64_t off = (int64_t)kt * 2048;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                r.q[(2 * j + s) & 3] = *reinterpret_cast<const v4u*>(bp[j] + off + s * 1024);
    }
}

template <int WQ>
__device__ __forceinline__ bf16x8_t b_frag(const BStep<WQ>& r, int j, int s) {
    v4u v;
    if (WQ == 1) {
        // the piece made opaque here, so that each fragment is widened where it
        // is used rather than all of them ahead (registers the loop lacks)
        v4u w = r.q[j & 1];
        asm volatile("" : "+v"(w));
        const unsigned w0 = s ? w.z : w.x, w1 = s ? w.w : w.y;
        v = v4u{i8pair_to_bf16(w0, 0), i8pair_to_bf16(w0, 16), i8pair_to_bf16(w1, 0), i8pair_to_bf16(w1, 16)};
    } else {
        v = r.q[(2 * j + s) & 3];
    }
    return __builtin_bit_cast(bf16x8_t, v);
}

// A: wavefront w moves rows [32w, 32w+32) of the K-step (4 x 1 KB); within
// each 1 KB (8 rows of 128 B) lane l lands in row l/8, physical chunk l%8, and
// so fetches logical chunk (l%8) ^ a_swz(row).
// The waits below count loads in issue order, so the compiler may not move
// any other load across these: compiler-only memory barriers on both sides.
__device__ __forceinline__ void a_dma(const char* const (&ap)[kADma], int kt, uint16_t* stage, int wave) {
    const int64_t off = (int64_t)kt * BK * 2;
    asm volatile("" ::: "memory");
#pragma unroll
    for (int q = 0; q < kADma; ++q)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(ap[q] + off),
                                         (lds_void_t*)(stage + (wave * kADma * 8 + q * 8) * BK), 16, 0, 0);
    asm volatile("" ::: "memory");
}

// MFMAs of one K-step over the first NSL 16-row slabs: A fragments from LDS
// (row 16 i + l % 16, k chunk 2 (l / 16) + s: the same k as the B fragment of
// the lane), B from registers. Slabs go in groups of four: the group's A
// fragments are read before its MFMAs, so that the LDS latency is paid once
// per group rather than once per fragment.
template <int WQ, int NSL>
__device__ __forceinline__ void mma_step(const uint16_t* As, const BStep<WQ>& rb, int lane,
                                         f32x4_t (&acc)[kSlabs][2]) {
    if (WQ == 2) {
        // E4M3: one 16x16x128 MFMA per slab and column tile. Lane l gives the
        // 32 codes at k = 16 (l / 16) .. + 15 of each 64-wide half of the
        // K-step, for A (chunks l / 16 and 4 + l / 16 of the row) and B (its
        // piece of tiles 2 kt and 2 kt + 1) alike, so the products pair the same k.
        const v8i b0 = cat8(rb.q[0], rb.q[1]), b1 = cat8(rb.q[2], rb.q[3]);
        const int c0 = lane >> 4, c1 = 4 + (lane >> 4);
        // slabs in pairs: an A fragment is twice a bf16 one, so a pair holds
        // the registers a group of four does there
#pragma unroll
        for (int g = 0; g < NSL; g += 2) {
            v4u a0[2], a1[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = (g + i) * 16 + (lane & 15);
                a0[i] = *reinterpret_cast<const v4u*>(As + swz(r, c0));
                a1[i] = *reinterpret_cast<const v4u*>(As + swz(r, c1));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const v8i a = cat8(a0[i], a1[i]);
                // operand formats 0 (E4M3) and unit E8M0 scales (127 = 2^0)
                acc[g + i][0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b0, acc[g + i][0], 0, 0, 0,
                                                                                 127, 0, 127);
                acc[g + i][1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b1, acc[g + i][1], 0, 0, 0,
                                                                                 127, 0, 127);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        return;
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const bf16x8_t b0 = b_frag<WQ>(rb, 0, s), b1 = b_frag<WQ>(rb, 1, s);
        const int c = (lane >> 4) * 2 + s;
#pragma unroll
        for (int g = 0; g < NSL; g += 4) {
            bf16x8_t af[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const bf16x8_t*>(As + swz((g + i) * 16 + (lane & 15), c));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[g + i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b0, acc[g + i][0], 0, 0, 0);
                acc[g + i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], b1, acc[g + i][1], 0, 0, 0);
            }
            // DS reads first, then the MFMAs, in one scheduling group each
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
    }
}

// LDS of a workgroup: kDepth distinct stages of A (distinct objects, so that
// the compiler can tell which stage a pending direct load writes).
struct Lds {
    uint16_t* a[kDepth];  // after the K loop, also the epilogue's staging
    float* rw;            // down: router weight of each row of the tile
};

// s_waitcnt vmcnt(n) lgkmcnt(0) (vmcnt split over bits 3:0 and 15:14)
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// The K loop over NSL slabs (NSL = 0: a wavefront with no valid column still
// moves its share of A and keeps the barriers, but loads no B).
//
// Pipeline, distance kDepth - 1 for both operands: step k issues A(k+3) into
// the LDS stage read at step k-1 and B(k+3) into the register slot read at
// step k-1, then runs the MFMAs of step k. Loads complete in issue order, so
// before step k the wavefront waits until at most the loads of the two later
// steps are pending: then its A(k) and B(k) have landed. A barrier then
// publishes every wavefront's A share and frees the stage read at step k-1.
// (A shallower A distance would drain the B ring too: waiting for an A load
// also waits for every B load issued before it.) a_dma and a compiler memory
// barrier after b_load pin the order of the loads against compiler
// scheduling: a B load sunk below the MFMAs (to reuse the registers they
// read) leaves the compiler unsure, across the loop's back edge, which loads
// a register still waits for, and it then waits for all of them once per
// unrolled group, draining the ring. Loads past the last K-step repeat the
// last one, so every step issues the same loads.
template <int WQ, int NSL, bool ADMA>
__device__ __forceinline__ void k_loop(const char* const (&ap)[kADma], const char* const (&bp)[2], int nk, int nkt,
                                       const Lds& L, int wave, int lane, f32x4_t (&acc)[kSlabs][2]) {
    constexpr int kA = ADMA ? kADma : 0;
    constexpr int kB = NSL > 0 ? kBLoads<WQ> : 0;
    constexpr int kWait = wait_vm_lgkm0((kDepth - 2) * (kA + kB));
    static_assert((kDepth - 2) * (kA + kB) < 64, "vmcnt range");
    static_assert(kDepth == 4, "four stages and slots below");
    const int last = nk - 1;
    BStep<WQ> rb0, rb1, rb2, rb3;
    uint16_t* const S0 = L.a[0];
    uint16_t* const S1 = L.a[1];
    uint16_t* const S2 = L.a[2];
    uint16_t* const S3 = L.a[3];
    // (the prologue's B loads in step order too: with rb0 issued last, the
    // compiler's wait for it at the first step of every unrolled group would
    // drain the ring)
    if (ADMA) a_dma(ap, 0, S0, wave);
    if (NSL > 0) b_load<WQ>(bp, 0, nkt, rb0);
    asm volatile("" ::: "memory");
    if (ADMA) a_dma(ap, min(1, last), S1, wave);
    if (NSL > 0) b_load<WQ>(bp, min(1, last), nkt, rb1);
    asm volatile("" ::: "memory");
    if (ADMA) a_dma(ap, min(2, last), S2, wave);
    if (NSL > 0) b_load<WQ>(bp, min(2, last), nkt, rb2);
    asm volatile("" ::: "memory");
#define MOE_GEMM_STEP(U, SA, RB, SN, RN)                                    \
    __builtin_amdgcn_s_waitcnt(kWait);                                      \
    raw_barrier();                                                          \
    if (ADMA) a_dma(ap, min(kt + (U) + kDepth - 1, last), SN, wave);        \
    if (NSL > 0) {                                                          \
        b_load<WQ>(bp, min(kt + (U) + kDepth - 1, last), nkt, RN);        \
        asm volatile("" ::: "memory");                                      \
        if (kt + (U) < nk) mma_step<WQ, NSL>(SA, RB, lane, acc);          \
    }
    for (int kt = 0; kt < nk; kt += kDepth) {
        MOE_GEMM_STEP(0, S0, rb0, S3, rb3)
        MOE_GEMM_STEP(1, S1, rb1, S0, rb0)
        MOE_GEMM_STEP(2, S2, rb2, S1, rb1)
        MOE_GEMM_STEP(3, S3, rb3, S2, rb2)
    }
#undef MOE_GEMM_STEP
    __builtin_amdgcn_s_waitcnt(7 << 4);  // vmcnt(0) lgkmcnt(0): no load still in flight
    raw_barrier();
}

template <int MODE, int WQ>
__device__ __forceinline__ void gemm_block(const GemmArgs& p, int b, const Lds& L) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int wn = wave;
    const int n_nt = n_tiles_of<MODE>(p);

    // XCD-aware mapping (gemm_expert_blocks): the routed experts' tile of this
    // block comes precomputed from the grouping; the dense problem's units are
    // shared out as dense_groups describes.
    int group = 0, row0, rows_valid, nt;
    if (p.tiles) {
        const int2 te = p.tiles[b];
        if (te.y < 0) return;
        row0 = te.x;
        group = te.y & 511;
        rows_valid = (te.y >> 9) & 511;
        nt = te.y >> 18;
    } else {
        const int m_total = (p.M_dense + BM - 1) / BM;
        const int units = m_total * n_nt, share = (units + kXcds - 1) / kXcds;
        const int u = (b % kXcds) * share + b / kXcds;  // block b runs on XCD b % kXcds
        if (b / kXcds >= share || u >= units) return;
        const int gm = dense_groups<MODE>(p), mc = (m_total + gm - 1) / gm;
        const int mg = u / (mc * n_nt), r = u - mg * mc * n_nt;  // every group but the last holds mc
        const int m_in = min(mc, m_total - mg * mc);
        nt = r / m_in;
        const int mt = mg * mc + (r - nt * m_in);
        row0 = mt * BM;
        rows_valid = min(BM, p.M_dense - row0);
    }

    f32x4_t acc[kSlabs][2];
#pragma unroll
    for (int i = 0; i < kSlabs; ++i) acc[i][0] = acc[i][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // valid 16-row slabs, rounded up to a multiple of 4 (the extra slabs hold
    // repeated rows and are never stored); 0 for a gate/up wavefront past the
    // last h column
    const int n_slabs = min(kSlabs, (rows_valid + 15) / 16);
    int nsl = (n_slabs + 3) / 4 * 4;
    if (MODE == MODE_GATEUP && nt * kHalfN + wn * 16 >= p.n_out) nsl = 0;
    // K-steps: 64 values (bf16, int8), or 128 E4M3 codes; B tiles are 64 wide
    const int nkt = p.K / BK;
    const int nk = WQ == 2 ? (nkt + 1) / 2 : nkt;

    // sources: B fragments of this lane (column l % 16 of tiles 0 and 1, k from
    // 16 (l / 16)) in the tiled layout; A rows of this wavefront's DMA share
    const char* bp[2];
    {
        const int esz = WQ ? 1 : 2;
        const char* B = (const char*)p.B + (int64_t)group * p.b_group_stride * esz;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
            bp[jj] = B + (int64_t)b_tile<MODE>(p, nt, wn, jj) * nkt * (esz * 1024) + lane * 16;
    }
    const char* ap[kADma];
#pragma unroll
    for (int q = 0; q < kADma; ++q) {
        const int r = wave * kADma * 8 + q * 8 + (lane >> 3);
        const int c = (lane & 7) ^ a_swz(r);
        const int rr = min(r, rows_valid - 1);  // rows past the tile end repeat a valid row
        const int64_t arow = p.a_rows ? p.a_rows[row0 + rr] : (int64_t)(row0 + rr);
        // a row: lda bf16 values, or lda bytes of E4M3 codes; its 16-byte chunk c of a K-step
        ap[q] = reinterpret_cast<const char*>(p.A) + arow * p.lda * (WQ == 2 ? 1 : 2) + c * 16;
    }
    // epilogue operands, loaded now so that their latency hides behind the K
    // loop: 1-byte formats' column scales of this lane's columns, router weight of row tid
    const int col_l = lane & 15;
    float sc0 = 1.f, sc1 = 1.f, row_wt = 1.f;
    if (WQ) {
        const float* bs = p.b_scale + (int64_t)group * p.scale_group_stride;
        if (MODE == MODE_GATEUP) {
            const int hc = min(nt * kHalfN + wn * 16 + col_l, p.n_out - 1);
            sc0 = bs[hc];
            sc1 = bs[p.up_off + hc];
        } else {
            sc0 = bs[nt * BN + wn * 32 + col_l];
            sc1 = bs[nt * BN + wn * 32 + 16 + col_l];
        }
    }
    if (MODE == MODE_DOWN && !p.Cf && tid < BM)
        row_wt = tid >= rows_valid ? 0.f : p.row_w ? p.row_w[row0 + tid] : 1.f;
    // E4M3 gate/up: the per-token scale of each A row
    if (MODE == MODE_GATEUP && WQ == 2 && tid < BM) {
        const int rr = min(tid, rows_valid - 1);
        const int64_t arow = p.a_rows ? p.a_rows[row0 + rr] : (int64_t)(row0 + rr);
        row_wt = p.a_scale[arow];
    }
    // A rows the MFMAs read: the valid slabs rounded up to groups of four (the
    // same for every wavefront); a wavefront whose 32 DMA rows all lie past them
    // moves no A (its wait counts are its own loads, so they differ by template)
    const int rows_read = (n_slabs + 3) / 4 * 64;
    const bool adma = wave * kADma * 8 < rows_read;
#define MOE_K_LOOP(N)                                                      \
    do {                                                                   \
        if (adma) k_loop<WQ, N, true>(ap, bp, nk, nkt, L, wave, lane, acc); \
        else k_loop<WQ, N, false>(ap, bp, nk, nkt, L, wave, lane, acc);     \
    } while (0)
    switch (nsl) {  // uniform per wavefront
        case 0: MOE_K_LOOP(0); break;
        case 4: MOE_K_LOOP(4); break;
        case 8: MOE_K_LOOP(8); break;
        case 12: MOE_K_LOOP(12); break;
        default: MOE_K_LOOP(16); break;
    }
#undef MOE_K_LOOP

    // epilogue: acc[i][jj][v] is C[row = 16 i + 4 (lane>>4) + v][column tile jj, lane&15]
    if (MODE == MODE_GATEUP) {
        // the h tile [BM][128] bf16, rows 128 h .. + 128 staged in A stage h (32 KB each)
        const int hl = wn * 16 + col_l;  // column within the 128-wide h tile
        if (WQ == 2) {
            if (tid < BM) L.rw[tid] = row_wt;
            lds_barrier();
        }
#pragma unroll
        for (int i = 0; i < kSlabs; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = i * 16 + (lane >> 4) * 4 + v;
                const float rs = WQ == 2 ? L.rw[r] : 1.f;
                const float g = acc[i][0][v] * sc0 * rs, u = acc[i][1][v] * sc1 * rs;
                L.a[i >> 3][(r & 127) * kHalfN + hl] = f32_to_bf16(gelu_tanh(g) * u);
            }
        lds_barrier();
        const int h_valid = min(kHalfN, p.n_out - nt * kHalfN);
#pragma unroll
        for (int q = 0; q < BM * kHalfN / 8 / kThreads; ++q) {
            const int c = tid + kThreads * q, r = c >> 4, cc = c & 15;
            if (r < rows_valid && cc * 8 < h_valid)
                *reinterpret_cast<uint4*>(p.C + (int64_t)(row0 + r) * p.ldc + nt * kHalfN + cc * 8) =
                    *reinterpret_cast<const uint4*>(L.a[r >> 7] + (r & 127) * kHalfN + cc * 8);
        }
    } else if (p.Cf) {
        // fp32 output straight from the accumulators (16 lanes write 64 contiguous bytes)
#pragma unroll
        for (int i = 0; i < kSlabs; ++i)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int r = i * 16 + (lane >> 4) * 4 + v;
                if (r < rows_valid) {
                    float* dst = p.Cf + (int64_t)(row0 + r) * p.ldc + nt * BN + wn * 32 + col_l;
                    dst[0] = acc[i][0][v];
                    dst[16] = acc[i][1][v];
                }
            }
    } else {
        // bf16 rows times the router weight: rows 64 h .. + 64 staged in A stage h (32 KB each)
        if (tid < BM) L.rw[tid] = row_wt;
        lds_barrier();
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int cl = wn * 32 + jj * 16 + col_l;
            const float sc = jj ? sc1 : sc0;
#pragma unroll
            for (int i = 0; i < kSlabs; ++i)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int r = i * 16 + (lane >> 4) * 4 + v;
                    L.a[i >> 2][(r & 63) * BN + cl] = f32_to_bf16(acc[i][jj][v] * sc * L.rw[r]);
                }
        }
        lds_barrier();
#pragma unroll
        for (int q = 0; q < BM * BN / 8 / kThreads; ++q) {
            const int c = tid + kThreads * q, r = c >> 5, cc = c & 31;
            if (r < rows_valid)
                *reinterpret_cast<uint4*>(p.C + (int64_t)(row0 + r) * p.ldc + nt * BN + cc * 8) =
                    *reinterpret_cast<const uint4*>(L.a[r >> 6] + (r & 63) * BN + cc * 8);
        }
    }
}

template <int MODE, int WQ_0, int WQ_1>
__global__ __launch_bounds__(kThreads) void gemm_kernel(GemmArgs p0, GemmArgs p1, int split) {
    // four LDS stages of A (256 x 64 bf16, 32 KB each; after the K loop, the
    // epilogue's staging) and the tile's router weights
    __shared__ __attribute__((aligned(16))) uint16_t st0[kAStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t st1[kAStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t st2[kAStageElems];
    __shared__ __attribute__((aligned(16))) uint16_t st3[kAStageElems];
    __shared__ float rw[BM];
    const Lds L{{st0, st1, st2, st3}, rw};
    const int b = blockIdx.x;
    if (b < split) gemm_block<MODE, WQ_0>(p0, b, L);
    else gemm_block<MODE, WQ_1>(p1, b - split, L);
}

// first and second problem back to back in one grid (each a whole number of
// XCD rounds, so block b of either runs on XCD b % 8)
template <int MODE, int WQ_0, int WQ_1>
hipError_t launch(const GemmArgs& first, const GemmArgs* second, hipStream_t stream) {
    const int b0 = blocks_of<MODE>(first);
    const int b1 = second ? blocks_of<MODE>(*second) : 0;
    if (b0 + b1 <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<MODE, WQ_0, WQ_1>), dim3((unsigned)(b0 + b1)), dim3(kThreads),
                       0, stream, first, second ? *second : first, b0);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ dense,
                                                      const uint16_t* __restrict__ rows,
                                                      const int32_t* __restrict__ inv_row, int T,
                                                      int H, int K, uint16_t* __restrict__ y) {
    const int hc = H / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * hc) return;
    const int64_t t = i / hc;
    const int c = (int)(i - t * hc) * 8;
    int q[kMaxTopKGemm];
#pragma unroll
    for (int k = 0; k < kMaxTopKGemm; ++k) q[k] = inv_row[t * K + min(k, K - 1)];
    // the rows and the dense output are read once: non-temporal loads (at the
    // skewed T=16384, 1 GB a launch, they measured 15% faster than plain ones)
    typedef float f4v __attribute__((ext_vector_type(4)));
    uint4 rv[kMaxTopKGemm];
#pragma unroll
    for (int k = 0; k < kMaxTopKGemm; ++k) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(rows + (int64_t)q[k] * H + c));
        rv[k] = make_uint4(v.x, v.y, v.z, v.w);
    }
    const f4v e0 = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(dense + t * H + c));
    const f4v e1 = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(dense + t * H + c + 4));
    const float4 d0 = make_float4(e0.x, e0.y, e0.z, e0.w), d1 = make_float4(e1.x, e1.y, e1.z, e1.w);
    float o[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
    for (int k = 0; k < kMaxTopKGemm; ++k) {
        if (k < K) {
            float f[8];
            unpack8(rv[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += f[e];
        }
    }
    *reinterpret_cast<uint4*>(y + t * H + c) = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                                          pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
}

}  // namespace

// wq: the experts' weight format (0 bf16, 1 int8, 2 E4M3); the dense problem is bf16
hipError_t launch_gemm_gateup(const GemmArgs& experts, const GemmArgs* dense, int wq,
                              hipStream_t stream) {
    // the dense problem first: its tiles hold full 256-row M-tiles and run
    // longest, so the shorter expert tiles fill the end of the launch
    if (!dense) {
        if (wq == 2) return launch<MODE_GATEUP, 2, 2>(experts, nullptr, stream);
        return wq ? launch<MODE_GATEUP, 1, 1>(experts, nullptr, stream)
                  : launch<MODE_GATEUP, 0, 0>(experts, nullptr, stream);
    }
    if (wq == 2) return launch<MODE_GATEUP, 0, 2>(*dense, &experts, stream);
    return wq ? launch<MODE_GATEUP, 0, 1>(*dense, &experts, stream)
              : launch<MODE_GATEUP, 0, 0>(*dense, &experts, stream);
}
hipError_t launch_gemm_down(const GemmArgs& experts, const GemmArgs* dense, int wq,
                            hipStream_t stream) {
    // the dense problem first: its blocks run a longer reduction (alone, its
    // few 256-row tiles would leave most of the chip idle)
    if (!dense) {
        if (wq == 2) return launch<MODE_DOWN, 2, 2>(experts, nullptr, stream);
        return wq ? launch<MODE_DOWN, 1, 1>(experts, nullptr, stream)
                  : launch<MODE_DOWN, 0, 0>(experts, nullptr, stream);
    }
    if (wq == 2) return launch<MODE_DOWN, 0, 2>(*dense, &experts, stream);
    return wq ? launch<MODE_DOWN, 0, 1>(*dense, &experts, stream)
              : launch<MODE_DOWN, 0, 0>(*dense, &experts, stream);
}
hipError_t launch_combine(const float* dense_out, const uint16_t* rows, const int32_t* inv_row,
                          int T, int H, int K, uint16_t* y, hipStream_t stream) {
    const int64_t n = (int64_t)T * (H / 8);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       dense_out, rows, inv_row, T, H, K, y);
    return hipGetLastError();
}

}  // namespace moe
