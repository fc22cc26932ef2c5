// Every few-rows workgroup shape of one pass in a single launch (bf16).
//
// A batch that mixes window lengths (for instance the five forgetting-curve
// settings of the WAITS README's action table over one prompt: row blocks of
// fully weighted prompts beside heads of a few dozen processed rows) has
// heads on several workgroup shapes.  One launch per shape makes each wait
// for the previous one's tail, with most compute units idle; here the
// shapes' work items share one grid of 512-thread workgroups.  Segment s of
// the grid, [begin[s], end[s]), holds the items of shape s; the host chooses
// the segments' order.  A workgroup of a shape with fewer than 8 waves ends
// its other waves at once; the hardware barrier then waits only for the
// waves still running.  The LDS is the union of the shapes' layouts, so the
// launch holds as much LDS per workgroup as the largest shape alone.
//
// Shape s is FR_SHAPES[s] of the host plan: 0, 1, 2: 2, 4 and 8 waves of one
// 32-row tile; 3, 4: the 16-row-tile kernel with 3 and 4 tiles per wave;
// 5: 8 waves of two 32-row tiles (the row-block shape).
#pragma once

#include "device_common.hpp"
#include "few_rows.hpp"
#include "few_rows16.hpp"
#include "kernel_args.hpp"

namespace waits {

constexpr int FR_MULTI_SHAPES = 6;

struct FrMultiArgs {
  FrArgs f;                                     // f.tab.first unused
  int32_t begin[FR_MULTI_SHAPES];               // first workgroup of each shape's segment
  int32_t end[FR_MULTI_SHAPES];                 // one past its last (== begin: no items)
  int32_t first[FR_MULTI_SHAPES][MAXB + 1];     // first item of each sequence, per shape
};

template <int D>
union FrMultiLds {
  FrLds<bf16_t, D, 2, 1> s0;
  FrLds<bf16_t, D, 4, 1> s1;
  FrLds<bf16_t, D, 8, 1> s2;
  Fr16Lds<D, 3> s3;
  Fr16Lds<D, 4> s4;
  FrLds<bf16_t, D, 8, 2> s5;
};

template <int D, bool PASS2>
__global__ void __launch_bounds__(512)
few_rows_multi_kernel(const FrMultiArgs args) {
  __shared__ FrMultiLds<D> L;
  const int b = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  auto in = [&](int s) { return b >= args.begin[s] && b < args.end[s]; };
  if (in(5)) {
    few_rows_body<bf16_t, D, PASS2, 8, 2>(args.f, args.first[5], b - args.begin[5], L.s5);
  } else if (in(4)) {
    few_rows16_body<D, PASS2, 4>(args.f, args.first[4], b - args.begin[4], L.s4);
  } else if (in(3)) {
    few_rows16_body<D, PASS2, 3>(args.f, args.first[3], b - args.begin[3], L.s3);
  } else if (in(2)) {
    few_rows_body<bf16_t, D, PASS2, 8, 1>(args.f, args.first[2], b - args.begin[2], L.s2);
  } else if (in(1)) {
    if (wave < 4) few_rows_body<bf16_t, D, PASS2, 4, 1>(args.f, args.first[1], b - args.begin[1], L.s1);
  } else if (in(0)) {
    if (wave < 2) few_rows_body<bf16_t, D, PASS2, 2, 1>(args.f, args.first[0], b - args.begin[0], L.s0);
  }
}

}  // namespace waits
