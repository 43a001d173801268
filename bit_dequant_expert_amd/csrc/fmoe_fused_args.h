// fmoe_fused_args.h -- argument block of the one-launch layer kernel, shared
// by the host dispatch and the kernel.
#pragma once

#include <stdint.h>

#include "fmoe_internal.h"

namespace fmoe {

// Counter and flag block at the start of the workspace (520 lines of 256 B).
constexpr int kFusedCtrLines = 520;
constexpr size_t kFusedCtrBytes = (size_t)kFusedCtrLines * 256;

// Work-item sizes (4 waves per workgroup).  A gate/up part is UG rows of gate
// and of up per wave (one expert): UG = 4 when a lane reads one 16-byte
// segment of a hidden-size row, 2 when it reads two (register budget of two
// workgroups per CU).  A down part is kFusedUD row iterations per wave over
// every active expert.
constexpr int kFusedWaves = 4;
constexpr int kFusedUD = 1;
constexpr int kFusedMaxNormParts = 4 * 256;   // down parts the final norm sums
// Record area of the one-token layer kernel (fmoe_tok1.h): the epoch line,
// then up to kTok1MaxE logit records, up to kTok1MaxI2/2 shared-expert SwiGLU
// records (two values each), up to kTok1MaxParts sum-of-squares records and
// the routed SwiGLU block records of up to kTok1MaxSlots images (4 bytes per
// element of the intermediate size in both code formats).
constexpr int kTok1MaxE = 2048;
constexpr int kTok1MaxParts = 1024;
constexpr int kTok1MaxSlots = 17;
constexpr int kTok1ImgBytesPerElem = 4;
constexpr int kTok1MaxI4 = 2048, kTok1MaxI2 = 4096;
constexpr size_t kTok1LogitOff = 256;
constexpr size_t kTok1SharedOff = kTok1LogitOff + 16 * (size_t)kTok1MaxE;
// Part records: one per down part (its sum of h^2), or, in the chained kernel,
// (d_rows + 3) / 3 per part (its d_rows values of h and their sum of squares),
// at most kTok1MaxPartRecs in all.
constexpr int kTok1MaxPartRecs = 3 * kTok1MaxParts;
constexpr size_t kTok1PartOff = kTok1SharedOff + 16 * (size_t)(kTok1MaxI2 / 2);
constexpr size_t kTok1ImgOff = kTok1PartOff + 16 * (size_t)kTok1MaxPartRecs;
constexpr size_t kTok1AreaBytes =
    (kTok1ImgOff + (size_t)kTok1MaxSlots * kTok1ImgBytesPerElem * kTok1MaxI2 + 255) / 256 * 256;

// Every workspace layout keeps its data past this head, which holds only
// counters that each call returns to zero and the one-token kernel's record
// area (self-checking records, never read as data by another call kind): a
// call of any kind never leaves data where another kind of call keeps its
// counters or records.
// Two record areas: the one-token kernel uses the first, the chained kernel
// alternates between both by layer.
constexpr size_t kWsReserved = kFusedCtrBytes + 2 * kTok1AreaBytes;
__host__ __device__ constexpr int fused_ug(int nsh) { return nsh == 1 ? 4 : 2; }
inline int fused_gu_rows(int H, int bits) { return kFusedWaves * fused_ug(segs_per_lane(H, bits)); }
inline int fused_d_rows(int I, int bits) { return kFusedWaves * kFusedUD * rows_per_iter(I, bits); }

struct FusedArgs {
  ExpertSrc src;
  const float* Wr;
  const float* wsg;
  const float* x;
  const float* resid;
  const float* gamma;
  float* h_out;
  float* y_out;
  float* moe_out;
  float* w_out;
  int32_t* idx_out;
  float eps;
  int H, I, E, k;
  double* lg64;      // [E+1]
  float* abuf;       // [(k+1) * I]  SwiGLU outputs, slot-major (slot 0 the shared expert)
  float* gh;         // [H]  gamma * h, read by the final norm
  float* partials;   // [nD]  sum of h^2 per down part
  int* dlist;        // [nD]  down parts deferred to the end of the queue
  int* ctr;          // counter and flag block (kFusedCtrBytes)
  int nGUs;          // gate/up parts per expert (I / gu_rows)
  int nD;            // down parts
  int nF;            // items: item f holds shared gate/up part f, routed gate/up
                     // part f (expert slot f / nGUs) and down part f
  int nRr;           // items holding router rows (rows f, f + nRr, ... below E;
                     // row E, the shared-expert gate, goes to item E mod nRr); set
                     // by the launcher to min(grid, E), so they are all first items
  int gu_rows;       // gate/up rows per part
  int d_rows;        // down rows per part
};

// Arguments of the one-token layer kernel with self-checking records (fmoe_tok1.h).
struct Tok1Args {
  // The first 64 bytes hold what the kernel's first loads need (they are
  // preloaded into scalar registers at wave launch where the hardware does so).
  const float* x;
  const float* Wr;
  uint8_t* area;      // record area (kTok1AreaBytes)
  const float* wsg;
  const uint8_t* slabs;
  int64_t stride;     // bytes between expert slabs; slab E is the shared expert
  int H, I, E, k;
  // the rest
  int64_t off[9];     // section offsets within a slab
  const float* resid;
  const float* gamma;
  float* h_out;
  float* y_out;
  float* moe_out;
  float* w_out;
  int32_t* idx_out;
  float eps;
  int* timeout;       // the workspace's timeout word
  int nGUs;           // gate/up parts per expert (I / gu_rows)
  int nD;             // down parts (H / d_rows)
  int gu_rows, d_rows;
  uint64_t spin_ticks;  // wall-clock limit of one wait (100 MHz ticks)
  int stall_part;     // >= 0: that down part never publishes its sum (test of the timeout path)
  uint64_t* trace;    // phase trace (builds with FMOE_TRACE only): kTok1TraceEvents per workgroup
};
constexpr int kTok1TraceEvents = 16;

// Layers of one launch of the chained one-token kernel (fmoe_chain.h): the
// per-layer pointers travel as kernel arguments.
constexpr int kTok1MaxChain = 64;
struct Tok1ChainLayer {
  const float* Wr;
  const float* wsg;
  const float* gamma;
  const uint8_t* slabs;
};
struct Tok1Chain {
  Tok1ChainLayer layer[kTok1MaxChain];
  int n;
};

// Arguments of the one-launch single-expert FFN.
struct Expert1Args {
  const uint8_t *gq, *gs, *gb;   // gate [I x H]: codes, scales, biases
  const uint8_t *uq, *us, *ub;   // up   [I x H]
  const uint8_t *dq, *ds, *db;   // down [H x I]
  const float* x;                // [H]
  float* y;                      // [H]
  uint8_t* img;                  // wimg_bytes(I, bits): the SwiGLU output
  int* ctr;                      // counter block (kFusedCtrBytes)
  int H, I;
  int nGU, gu_rows;              // gate/up parts and their rows
  int nD, d_rows;                // down parts and their rows
};

}  // namespace fmoe
