// LDS layout of the window branch on the fp16 matrix cores (one 128-query
// block), shared by local_mfma_kernel and the clustering launch that runs the
// window blocks beside the Lloyd iterations (kmeans_slice.hip); the body
// itself is local_mfma_body.inc.
#pragma once
#include <type_traits>
#include "launch.h"
#include "mfma_split.h"

namespace ca {
namespace {

constexpr int kMRows = 160;                  // 16 halo + 128 + 16 halo key rows
constexpr int kMPlane = kMRows * kD * 2;     // bytes of one fp16 plane
constexpr int kMPlaneE = kMPlane / 2;
constexpr int kMOffV = 2 * kMPlane;
constexpr int kMLds = 4 * kMPlane;           // 81,920 B: two workgroups per CU
constexpr int kMChunks = kMRows * kD / 8;    // 8-element chunks per staged tensor
constexpr int kMItems = (kMChunks + kThreads - 1) / kThreads;
constexpr int kTabRows = 16;                 // V^cent table in LDS for Kc <= 16
constexpr int kTabStride = kD + 4;           // floats per table row (bank spread)

}  // namespace

}  // namespace ca
