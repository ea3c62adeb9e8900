// og_api.hip -- the C ABI of libog (declared in include/og.h): argument
// checks, the choice of kernel and tile from the shape alone, and launches.
//
// The tile is a function of the shape only, never of the device or of the
// load ("Matrix product and convolution kernels", section "Fixed chunks and
// thread independence"); the results do not depend on it anyway, because
// every output is summed whole, in one order, by one lane.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <string>

#include "og.h"
#include "og_kernels.hpp"
#include "og_launch.hpp"

namespace {

using namespace og::host;

thread_local hipStream_t t_stream = nullptr;
thread_local int t_variant = 0;
thread_local std::string t_error;

og_status fail(og_status code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  t_error = buf;
  return code;
}

og_status ok() {
  t_error.clear();
  return OG_OK;
}

constexpr int kMaxDevices = 64;
int g_device_state[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other

// The current device must be a gfx950.
og_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(OG_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(OG_ERR_DEVICE, "device index %d", dev);
  int st = __atomic_load_n(&g_device_state[dev], __ATOMIC_ACQUIRE);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(OG_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    __atomic_store_n(&g_device_state[dev], st, __ATOMIC_RELEASE);
    if (st < 0)
      return fail(OG_ERR_DEVICE, "device %d is %s; this library runs on gfx950 only", dev,
                  prop.gcnArchName);
  }
  if (st < 0) return fail(OG_ERR_DEVICE, "device %d is not gfx950", dev);
  return OG_OK;
}

og_status check_launch(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(OG_ERR_DEVICE, "%s launch: %s", what, hipGetErrorString(e));
  return ok();
}


// The shape the kernel choice sees: a group's product (M x N x K) and, for
// a convolution, the pixels of one output image and the window size (the
// lane and chain kernels tile columns per image for 1x1 and 3x3 windows).
struct Shape {
  int64_t M, N, K, groups;
  int64_t ohw;  // output pixels per image; 0 for a matrix product
  int64_t khw;  // KH * KW; 0 for a matrix product
  int ffam = 0;        // a convolution's family in the launch model (fast_family)
  double bytes = 0;    // bytes of the operands and the result, each counted once
  double halo_x = 0;   // halo kernel: thousands of input floats staged per block over its k
};

// Family of a convolution in the launch model: 1 a 3x3 window at stride 1,
// 4 a strided 3x3 window, 2 a 1x1 window read in place (stride 1, no
// padding), 6 a 1 x k window (k > 1: the 1-D convolutions), 3 any other
// window or a strided or padded 1x1 (gathered taps).
int fast_family(int64_t KH, int64_t KW, bool planes, int64_t strideH, int64_t strideW) {
  if (KH == 3 && KW == 3) return strideH == 1 && strideW == 1 ? 1 : 4;
  if (KH == 1 && KW > 1) return 6;
  return planes ? 2 : 3;
}
// Family of a matrix product: 5 from 2^32 multiply-adds up (sizes where the
// large tiles' time per block decides; one fit over all sizes overrated the
// 64 x 64 tile there), else 0.
int product_family(const Shape &s) {
  return (double)s.M * (double)s.N * (double)s.K >= 4294967296.0 ? 5 : 0;
}

// Launch time models, t in microseconds.  Fast mode: t = (c * K / 1000 + d
// + e * X) * rounds + o + b * bytes / 1e6, rounds = max(1, (1 - q) * x + q *
// ceil(x)) with x = blocks / cap, bytes those of the operands and the result
// each counted once, X (halo kernel only) the thousands of input floats a
// block stages over its k; (q, cap, c, d, o, b, e) per variant and family
// (fast_family, product_family), cap a multiple of 256 blocks (one or more
// per compute unit), fitted by least squares on the relative error to 457
// shapes (477 in exact mode), each launched on every variant on the MI355X
// (ResNet-50's
// convolutions at batch 1, 2, 3, 4, 5, 6, 8, 12 and 16, MobileNetV3-large's
// ungrouped ones at batch 1, 2, 4, 6 and 8, twelve 3x3 convolutions of other
// widths, 72 seeded random matrix products up to 2048 x 2900 x 2300, 36
// products of a language model's sizes (4096^3, 512 x 11008 x 4096,
// 1 x 4096 x 4096 and 33 seeded ones of m = 1..4096, n = 1024..11008,
// k = 1024..8192), 20 seeded 1-D convolutions and, in exact mode, 20
// products with unaligned rows): mean error 4.2 % (exact 3.9 %).  Variants 26..28 and
// 31..33 are the halo kernel, 29 and 30 the panel kernel.
struct ModelCost {
  int variant, fam;
  double q, cap, c, d, o, b, e;
};
constexpr ModelCost kFastCosts[] = {
    {2, 0, 0, 256, 130.323, 9.416, 0.000, 0.0239, 0.0000},
    {2, 1, 0, 256, 200.488, 0.000, 9.607, 0.0977, 0.0000},
    {2, 2, 0.75, 256, 135.149, 0.000, 8.754, 0.0683, 0.0000},
    {2, 3, 0.75, 256, 191.331, 4.963, 9.518, 0.0000, 0.0000},
    {2, 4, 1, 256, 198.851, 0.829, 9.278, 0.0386, 0.0000},
    {2, 5, 0.75, 256, 128.304, 2.595, 17.525, 0.0000, 0.0000},
    {2, 6, 0.75, 256, 201.719, 0.000, 9.362, 0.0000, 0.0000},
    {3, 0, 0, 256, 70.055, 5.914, 0.000, 0.0390, 0.0000},
    {3, 1, 0.5, 256, 106.661, 1.239, 5.154, 0.0499, 0.0000},
    {3, 2, 0.75, 256, 74.927, 0.448, 5.102, 0.0654, 0.0000},
    {3, 3, 0.75, 256, 103.345, 0.178, 8.299, 0.0000, 0.0000},
    {3, 4, 0.25, 256, 106.345, 2.227, 3.966, 0.0247, 0.0000},
    {3, 5, 0.75, 256, 67.837, 0.000, 11.640, 0.0000, 0.0000},
    {3, 6, 0, 256, 102.707, 0.000, 7.815, 0.0000, 0.0000},
    {4, 0, 0.5, 256, 39.546, 2.475, 1.766, 0.0000, 0.0000},
    {4, 1, 0.5, 256, 76.180, 0.000, 5.792, 0.0000, 0.0000},
    {4, 2, 0.5, 256, 44.865, 0.483, 3.795, 0.0623, 0.0000},
    {4, 3, 0.5, 256, 72.451, 0.000, 7.765, 0.0000, 0.0000},
    {4, 4, 0.75, 256, 76.090, 0.714, 4.108, 0.0483, 0.0000},
    {4, 5, 0.5, 256, 34.477, 0.000, 12.049, 0.1135, 0.0000},
    {4, 6, 0.5, 256, 66.137, 0.000, 10.942, 0.0000, 0.0000},
    {5, 0, 0.25, 256, 45.745, 2.829, 1.379, 0.0000, 0.0000},
    {5, 1, 0.5, 256, 117.752, 0.000, 5.240, 0.0000, 0.0000},
    {5, 2, 0.5, 256, 54.768, 0.387, 3.801, 0.0375, 0.0000},
    {5, 3, 0.5, 256, 107.044, 0.000, 8.889, 0.0000, 0.0000},
    {5, 4, 0.75, 256, 116.785, 1.327, 4.345, 0.0067, 0.0000},
    {5, 5, 0.5, 256, 36.621, 0.000, 10.466, 0.1963, 0.0000},
    {5, 6, 1, 512, 123.158, 0.000, 0.000, 0.5882, 0.0000},
    {6, 0, 0.75, 768, 15.713, 0.884, 1.995, 0.0458, 0.0000},
    {6, 1, 0.75, 768, 16.692, 0.000, 1.079, 0.0000, 0.0000},
    {6, 2, 0.5, 768, 14.497, 0.741, 2.710, 0.1789, 0.0000},
    {6, 3, 0.25, 768, 20.135, 4.491, 2.202, 0.0000, 0.0000},
    {6, 4, 0.5, 512, 17.816, 0.000, 3.089, 0.5236, 0.0000},
    {6, 5, 0.25, 1536, 31.162, 0.200, 0.309, 0.1142, 0.0000},
    {6, 6, 0, 512, 26.780, 0.000, 7.047, 2.3461, 0.0000},
    {7, 0, 0.75, 768, 18.099, 0.981, 1.964, 0.0518, 0.0000},
    {7, 1, 0.5, 768, 19.233, 0.000, 3.427, 0.0000, 0.0000},
    {7, 2, 0.5, 768, 17.275, 0.730, 2.542, 0.1325, 0.0000},
    {7, 3, 0.5, 512, 15.281, 2.631, 5.843, 0.0000, 0.0000},
    {7, 4, 0.75, 512, 20.614, 0.000, 3.038, 0.2773, 0.0000},
    {7, 5, 0.25, 768, 18.305, 0.000, 2.165, 0.1467, 0.0000},
    {7, 6, 0, 512, 29.051, 0.000, 7.635, 0.9218, 0.0000},
    {8, 0, 0.5, 512, 22.278, 0.478, 2.801, 0.0205, 0.0000},
    {8, 1, 0.25, 512, 23.173, 0.000, 4.585, 0.0000, 0.0000},
    {8, 2, 0.75, 768, 23.794, 0.559, 2.533, 0.1622, 0.0000},
    {8, 3, 0.75, 512, 20.253, 2.175, 5.834, 0.0000, 0.0000},
    {8, 4, 0.5, 512, 26.950, 0.000, 3.092, 0.1817, 0.0000},
    {8, 5, 0.25, 768, 27.693, 0.000, 3.876, 0.0769, 0.0000},
    {8, 6, 0, 512, 33.282, 0.000, 6.818, 0.3850, 0.0000},
    {9, 0, 1, 512, 31.443, 0.555, 3.053, 0.1385, 0.0000},
    {9, 1, 0, 2048, 29.070, 0.000, 0.000, 2.2430, 0.0000},
    {9, 2, 0.25, 512, 32.850, 0.000, 3.493, 0.1880, 0.0000},
    {9, 3, 0.5, 512, 32.239, 2.823, 4.915, 0.0000, 0.0000},
    {9, 4, 1, 512, 33.842, 0.000, 3.167, 0.3262, 0.0000},
    {9, 5, 0.25, 768, 46.021, 1.159, 16.829, 0.0000, 0.0000},
    {9, 6, 0.75, 768, 52.487, 0.000, 0.000, 0.5941, 0.0000},
    {10, 0, 1, 256, 6.029, 3.464, 1.564, 0.0388, 0.0000},
    {10, 1, 1, 256, 4.901, 3.893, 1.728, 0.0000, 0.0000},
    {10, 2, 1, 256, 5.242, 3.517, 1.783, 0.0000, 0.0000},
    {10, 3, 0.5, 512, 15.291, 13.569, 0.000, 0.4646, 0.0000},
    {10, 4, 1, 256, 3.995, 5.910, 1.106, 0.2118, 0.0000},
    {10, 5, 0.75, 512, 13.361, 5.341, 0.000, 0.0877, 0.0000},
    {11, 0, 1, 256, 5.120, 2.830, 1.475, 0.0196, 0.0000},
    {11, 1, 1, 256, 4.670, 3.157, 1.395, 0.0388, 0.0000},
    {11, 2, 1, 256, 4.418, 3.151, 1.633, 0.0748, 0.0000},
    {11, 3, 0.25, 1024, 25.793, 26.188, 0.000, 0.6820, 0.0000},
    {11, 4, 0.25, 256, 4.151, 4.723, 2.500, 0.0000, 0.0000},
    {11, 5, 1, 1024, 21.637, 9.818, 0.000, 0.0945, 0.0000},
    {12, 0, 1, 512, 3.361, 1.286, 2.651, 0.0427, 0.0000},
    {12, 1, 1, 256, 2.418, 1.180, 3.373, 0.2280, 0.0000},
    {12, 2, 0.25, 512, 3.202, 1.303, 3.748, 0.0000, 0.0000},
    {12, 3, 0.25, 2048, 19.515, 11.629, 3.561, 0.0000, 0.0000},
    {12, 4, 0, 256, 2.172, 1.702, 5.833, 0.0851, 0.0000},
    {12, 5, 1, 2048, 12.993, 4.877, 0.000, 0.2869, 0.0000},
    {13, 0, 1, 256, 6.537, 3.431, 1.563, 0.0122, 0.0000},
    {13, 1, 1, 256, 6.099, 3.497, 1.653, 0.0184, 0.0000},
    {13, 2, 1, 256, 6.283, 3.381, 1.657, 0.0000, 0.0000},
    {13, 3, 0.25, 512, 13.675, 13.472, 0.000, 0.3762, 0.0000},
    {13, 4, 0.75, 256, 4.884, 5.693, 2.003, 0.2918, 0.0000},
    {13, 5, 0.5, 512, 13.553, 5.992, 2.127, 0.0387, 0.0000},
    {14, 0, 1, 256, 9.051, 5.091, 2.106, 0.0000, 0.0000},
    {14, 1, 1, 256, 9.956, 5.491, 1.711, 0.0059, 0.0000},
    {14, 2, 1, 256, 7.045, 4.813, 1.979, 0.0000, 0.0000},
    {14, 3, 1, 256, 9.661, 7.993, 1.251, 0.1966, 0.0000},
    {14, 4, 0.5, 256, 7.366, 12.874, 1.225, 0.0000, 0.0000},
    {14, 5, 0.5, 512, 17.904, 8.537, 9.580, 0.0000, 0.0000},
    {15, 0, 1, 256, 9.844, 5.089, 2.029, 0.0000, 0.0000},
    {15, 1, 1, 256, 10.682, 4.264, 1.699, 0.0083, 0.0000},
    {15, 2, 1, 256, 8.417, 4.706, 1.838, 0.0000, 0.0000},
    {15, 3, 1, 256, 9.672, 7.894, 1.268, 0.1412, 0.0000},
    {15, 4, 0.5, 256, 7.929, 11.879, 1.208, 0.0000, 0.0000},
    {15, 5, 0.5, 512, 19.903, 8.240, 7.554, 0.0000, 0.0000},
    {16, 0, 1, 256, 7.558, 4.265, 1.610, 0.0101, 0.0000},
    {16, 1, 1, 256, 8.624, 3.982, 1.709, 0.0000, 0.0000},
    {16, 2, 1, 256, 6.525, 4.078, 1.922, 0.0000, 0.0000},
    {16, 3, 0.75, 256, 7.535, 7.375, 0.000, 0.2893, 0.0000},
    {16, 4, 0.75, 256, 6.736, 7.941, 1.861, 0.1315, 0.0000},
    {16, 5, 0.25, 1024, 31.425, 14.504, 6.658, 0.0101, 0.0000},
    {17, 0, 0, 256, 234.886, 10.173, 0.000, 0.1016, 0.0000},
    {17, 1, 0, 256, 289.559, 0.000, 10.965, 0.1087, 0.0000},
    {17, 2, 0.5, 256, 238.070, 9.250, 0.336, 0.0620, 0.0000},
    {17, 3, 1, 256, 282.211, 15.870, 0.221, 0.0000, 0.0000},
    {17, 4, 1, 256, 289.389, 8.416, 1.934, 0.0936, 0.0000},
    {17, 5, 1, 256, 235.543, 2.906, 3.549, 0.1560, 0.0000},
    {17, 6, 0, 256, 290.399, 10.880, 0.000, 0.0609, 0.0000},
    {20, 0, 0.5, 256, 27.886, 0.000, 3.846, 0.0000, 0.0000},
    {20, 1, 0.25, 256, 45.603, 0.000, 5.908, 0.0000, 0.0000},
    {20, 2, 0.25, 256, 28.724, 0.412, 4.546, 0.0276, 0.0000},
    {20, 3, 0.5, 256, 36.809, 0.000, 8.740, 0.0000, 0.0000},
    {20, 4, 0.25, 256, 46.385, 0.497, 4.725, 0.0000, 0.0000},
    {20, 5, 0, 256, 18.735, 0.000, 19.760, 0.1959, 0.0000},
    {20, 6, 0.5, 512, 45.669, 0.000, 6.827, 0.4091, 0.0000},
    {26, 1, 1, 256, 3.851, 0.000, 5.334, 0.9905, 0.0996},
    {26, 4, 1, 256, 4.864, 2.845, 3.406, 0.3862, 0.0789},
    {27, 1, 0.5, 256, 6.921, 1.587, 3.198, 0.4847, 0.1870},
    {27, 4, 1, 256, 9.054, 4.701, 2.449, 0.1241, 0.0583},
    {28, 1, 1, 256, 9.804, 3.408, 1.789, 0.1367, 0.1023},
    {28, 4, 1, 256, 11.834, 5.310, 2.876, 0.3160, 0.0204},
    {29, 0, 0.25, 256, 9.927, 0.600, 3.310, 0.0004, 0.0000},
    {29, 2, 0.5, 256, 8.419, 1.002, 3.144, 0.0000, 0.0000},
    {29, 3, 0.75, 256, 9.878, 1.438, 4.119, 0.3371, 0.0000},
    {29, 5, 0, 768, 21.665, 2.872, 15.191, 0.0000, 0.0000},
    {30, 0, 0.25, 256, 15.926, 0.543, 3.436, 0.0000, 0.0000},
    {30, 2, 0.25, 256, 14.384, 1.044, 3.014, 0.0000, 0.0000},
    {30, 3, 0.75, 256, 13.387, 0.000, 4.620, 0.3017, 0.0000},
    {30, 5, 0.25, 256, 11.824, 0.674, 13.275, 0.0178, 0.0000},
    {31, 1, 0.75, 256, 1.398, 1.006, 5.167, 1.3164, 0.0990},
    {31, 4, 1, 256, 1.436, 2.956, 0.011, 2.2745, 0.0854},
    {32, 1, 1, 256, 5.531, 3.008, 1.193, 0.3708, 0.1009},
    {32, 4, 1, 256, 9.695, 6.701, 1.730, 0.8313, 0.0000},
    {33, 1, 0.5, 256, 3.929, 0.000, 6.217, 1.3628, 0.0856},
    {33, 4, 1, 256, 0.904, 1.573, 2.845, 2.8047, 0.0995},
};

// Exact mode: the same form and families, fitted the same way to the same
// shapes launched in exact mode (variants 14..16 run as 10, 13 and 11 there,
// and 2, 3 and 17 on the 64 x 128 or 128 x 128 tile, whose blocks their
// entries count; the panel kernel has no exact form; variant 9, whose eight
// rows per lane are VALU-bound in exact mode, is left out of the choice).
constexpr ModelCost kExactCosts[] = {
    {2, 0, 0.25, 256, 100.479, 0.000, 6.662, 0.0000, 0.0000},
    {2, 1, 0, 256, 237.327, 0.000, 7.563, 0.0000, 0.0000},
    {2, 2, 0, 256, 103.383, 0.000, 4.836, 0.0342, 0.0000},
    {2, 3, 0, 256, 227.415, 0.000, 10.788, 0.0000, 0.0000},
    {2, 4, 0, 256, 237.609, 2.834, 4.086, 0.0000, 0.0000},
    {2, 5, 0, 256, 58.375, 0.000, 30.472, 0.9348, 0.0000},
    {2, 6, 0.75, 512, 239.827, 0.000, 2.032, 0.5130, 0.0000},
    {3, 0, 0.25, 256, 100.493, 0.000, 6.662, 0.0000, 0.0000},
    {3, 1, 0, 256, 237.329, 0.000, 7.556, 0.0000, 0.0000},
    {3, 2, 0, 256, 103.364, 0.000, 4.839, 0.0350, 0.0000},
    {3, 3, 0, 256, 227.422, 0.000, 10.802, 0.0000, 0.0000},
    {3, 4, 0, 256, 237.574, 2.833, 4.089, 0.0000, 0.0000},
    {3, 5, 0, 256, 58.559, 0.000, 29.973, 0.9301, 0.0000},
    {3, 6, 0.5, 512, 239.132, 0.000, 2.159, 0.5582, 0.0000},
    {4, 0, 0.25, 256, 100.482, 0.000, 6.669, 0.0000, 0.0000},
    {4, 1, 0, 256, 151.018, 0.000, 6.039, 0.0000, 0.0000},
    {4, 2, 0, 256, 103.386, 0.000, 4.837, 0.0349, 0.0000},
    {4, 3, 0.5, 512, 141.624, 2.887, 5.247, 0.3364, 0.0000},
    {4, 4, 0, 256, 151.080, 0.736, 4.422, 0.0532, 0.0000},
    {4, 5, 0, 256, 58.658, 0.000, 29.888, 0.9283, 0.0000},
    {4, 6, 1, 512, 156.699, 0.000, 1.624, 0.3594, 0.0000},
    {5, 0, 0, 256, 108.860, 0.000, 6.733, 0.0000, 0.0000},
    {5, 1, 0, 512, 216.461, 0.000, 1.328, 0.8328, 0.0000},
    {5, 2, 1, 512, 118.186, 0.028, 4.241, 0.1464, 0.0000},
    {5, 3, 0.25, 512, 203.916, 0.489, 10.213, 0.2272, 0.0000},
    {5, 4, 0.5, 256, 215.736, 0.000, 6.273, 0.0000, 0.0000},
    {5, 5, 0, 256, 63.828, 0.000, 0.000, 1.1038, 0.0000},
    {5, 6, 0.5, 768, 217.771, 0.441, 1.019, 0.5805, 0.0000},
    {6, 0, 0.5, 768, 16.735, 0.634, 2.253, 0.0384, 0.0000},
    {6, 1, 0.25, 768, 19.610, 0.000, 4.462, 0.0000, 0.0000},
    {6, 2, 0.5, 768, 14.674, 0.586, 2.825, 0.1742, 0.0000},
    {6, 3, 0.5, 768, 20.707, 4.075, 1.083, 0.0000, 0.0000},
    {6, 4, 0.5, 512, 18.571, 0.000, 2.904, 0.6610, 0.0000},
    {6, 5, 0.25, 1536, 32.813, 0.003, 0.000, 0.1111, 0.0000},
    {6, 6, 0, 512, 26.770, 0.021, 8.432, 2.1005, 0.0000},
    {7, 0, 0.75, 768, 20.832, 0.697, 2.108, 0.0409, 0.0000},
    {7, 1, 0.5, 768, 22.475, 0.000, 4.213, 0.0000, 0.0000},
    {7, 2, 0.5, 768, 20.429, 0.557, 2.781, 0.1081, 0.0000},
    {7, 3, 0.25, 512, 15.714, 2.626, 6.937, 0.0000, 0.0000},
    {7, 4, 0.25, 512, 23.841, 0.000, 3.332, 0.2151, 0.0000},
    {7, 5, 0.5, 768, 22.349, 0.000, 0.000, 0.0533, 0.0000},
    {7, 6, 0, 512, 32.147, 0.232, 8.262, 0.6587, 0.0000},
    {8, 0, 0.5, 512, 30.537, 0.000, 3.270, 0.0349, 0.0000},
    {8, 1, 0.5, 512, 31.168, 0.000, 5.015, 0.0000, 0.0000},
    {8, 2, 0.75, 768, 32.286, 0.373, 2.846, 0.1809, 0.0000},
    {8, 3, 0.5, 768, 31.659, 6.956, 0.922, 0.0000, 0.0000},
    {8, 4, 0.5, 512, 34.199, 0.000, 3.295, 0.1827, 0.0000},
    {8, 5, 0.25, 768, 38.080, 0.000, 1.375, 0.1186, 0.0000},
    {8, 6, 1, 512, 49.443, 0.000, 0.000, 1.4596, 0.0000},
    {10, 0, 1, 256, 7.145, 3.368, 1.667, 0.0228, 0.0000},
    {10, 1, 1, 256, 5.908, 3.806, 1.812, 0.0693, 0.0000},
    {10, 2, 1, 256, 6.559, 3.584, 1.781, 0.0000, 0.0000},
    {10, 3, 0.5, 512, 15.522, 13.777, 0.000, 0.4231, 0.0000},
    {10, 4, 0.75, 256, 5.230, 5.068, 2.269, 0.1950, 0.0000},
    {10, 5, 0.5, 1024, 29.988, 11.778, 0.000, 0.0617, 0.0000},
    {11, 0, 1, 256, 6.437, 2.911, 1.671, 0.0159, 0.0000},
    {11, 1, 1, 256, 5.729, 3.097, 1.304, 0.0581, 0.0000},
    {11, 2, 1, 256, 5.866, 3.245, 1.705, 0.0724, 0.0000},
    {11, 3, 0.25, 1024, 25.921, 26.732, 0.000, 0.5407, 0.0000},
    {11, 4, 0.5, 256, 5.239, 4.136, 2.964, 0.0246, 0.0000},
    {11, 5, 0.25, 2048, 52.987, 20.691, 0.000, 0.1080, 0.0000},
    {12, 0, 0.75, 512, 4.013, 1.227, 3.345, 0.0711, 0.0000},
    {12, 1, 1, 256, 3.152, 1.188, 3.755, 0.0733, 0.0000},
    {12, 2, 0.25, 512, 3.691, 1.351, 3.962, 0.0759, 0.0000},
    {12, 3, 0.25, 1024, 9.803, 5.836, 5.034, 0.0000, 0.0000},
    {12, 4, 0.5, 256, 2.971, 1.611, 4.888, 0.0190, 0.0000},
    {12, 5, 1, 1536, 11.528, 3.147, 0.000, 0.1019, 0.0000},
    {13, 0, 1, 256, 9.521, 3.393, 1.692, 0.0028, 0.0000},
    {13, 1, 1, 256, 9.141, 3.439, 1.583, 0.0192, 0.0000},
    {13, 2, 1, 256, 8.833, 3.567, 1.709, 0.0000, 0.0000},
    {13, 3, 0.25, 512, 16.051, 13.456, 0.000, 0.3438, 0.0000},
    {13, 4, 0.75, 256, 8.159, 5.185, 2.304, 0.2008, 0.0000},
    {13, 5, 0.25, 1024, 38.282, 12.294, 6.192, 0.0324, 0.0000},
    {17, 0, 0.25, 256, 100.474, 0.000, 6.666, 0.0000, 0.0000},
    {17, 1, 0, 256, 237.316, 0.000, 7.630, 0.0000, 0.0000},
    {17, 2, 0, 256, 103.369, 0.000, 4.827, 0.0371, 0.0000},
    {17, 3, 0, 256, 227.411, 0.000, 10.801, 0.0000, 0.0000},
    {17, 4, 0, 256, 237.674, 2.833, 4.082, 0.0000, 0.0000},
    {17, 5, 0, 256, 58.654, 0.000, 29.703, 0.9287, 0.0000},
    {17, 6, 0.5, 512, 238.988, 0.000, 2.174, 0.5598, 0.0000},
    {20, 0, 1, 512, 58.419, 0.000, 3.556, 0.1433, 0.0000},
    {20, 1, 0.25, 512, 92.985, 0.000, 2.441, 0.9360, 0.0000},
    {20, 2, 1, 512, 58.484, 0.412, 4.382, 0.1826, 0.0000},
    {20, 3, 0.5, 512, 90.270, 0.106, 8.587, 0.0740, 0.0000},
    {20, 4, 0.75, 768, 91.113, 0.549, 3.833, 0.7017, 0.0000},
    {20, 5, 0.75, 512, 66.107, 0.000, 0.000, 0.0000, 0.0000},
    {20, 6, 0.75, 768, 95.802, 0.000, 4.013, 0.5598, 0.0000},
    {26, 1, 1, 512, 12.688, 0.000, 3.411, 1.3181, 0.2810},
    {26, 4, 1, 256, 8.422, 0.000, 7.430, 1.5041, 0.1361},
    {27, 1, 0.25, 256, 24.060, 0.000, 6.895, 1.1480, 0.1870},
    {27, 4, 1, 256, 29.871, 4.356, 2.579, 0.1697, 0.0508},
    {28, 1, 1, 256, 19.915, 3.055, 1.923, 0.2576, 0.0705},
    {28, 4, 1, 256, 19.400, 5.357, 2.877, 0.4001, 0.0545},
    {31, 1, 0.75, 256, 2.623, 0.872, 5.827, 1.4970, 0.0902},
    {31, 4, 1, 256, 0.838, 2.716, 0.108, 2.7199, 0.1151},
    {32, 1, 1, 256, 8.928, 2.576, 1.874, 0.1531, 0.0968},
    {32, 4, 1, 256, 11.020, 7.444, 2.139, 0.4554, 0.0000},
    {33, 1, 0.75, 256, 6.808, 0.000, 6.582, 1.4772, 0.0548},
    {33, 4, 1, 256, 1.900, 0.269, 2.809, 3.4030, 0.1332},
};

// Blocks of a launch of variant t (columns per image where that kernel tiles so).
int64_t launch_blocks(const Tile &t, const Shape &s) {
  const bool per_image = s.ohw > 0 && (s.khw == 1 || s.khw == 9) && (is_lane(t) || is_chain(t));
  int64_t bm = t.bm, bn = t.bn;
  if (t.variant == 12 && s.khw == 9) bm = 2, bn = 32;  // the 3x3 form of variant 12
  const int64_t ncol = per_image ? (s.N / s.ohw) * ceil_div(s.ohw, bn) : ceil_div(s.N, bn);
  return ceil_div(s.M, bm) * ncol * s.groups;
}

// Estimate of `variant` on a launch of `blocks` blocks in exact or fast mode
// (mode 2 uses the fast one); 1e300 where the variant has no entry for the
// shape's family.
double model_estimate(int mode, int variant, const Shape &s, int64_t blocks) {
  const int fam = s.khw == 0 ? product_family(s) : s.ffam;
  auto scan = [&](const auto &table) {
    for (const ModelCost &c : table) {
      if (c.variant != variant || c.fam != fam) continue;
      const double k = (double)(s.K > 0 ? s.K : 1);
      const double x = (double)blocks / c.cap;
      const double rounds = std::max(1.0, (1.0 - c.q) * x + c.q * std::ceil(x));
      return (c.c * 1e-3 * k + c.d + c.e * s.halo_x) * rounds + c.o + c.b * 1e-6 * s.bytes;
    }
    return 1e300;
  };
  return mode == OG_MODE_EXACT ? scan(kExactCosts) : scan(kFastCosts);
}

double estimate(const Tile &t, const Shape &s, int mode) {
  // exact mode runs variants 2, 3 and 17 on the 64 x 128 tile (128 x 128
  // with gathered taps; launch_kind): their launches have that tile's blocks
  if (mode == OG_MODE_EXACT && (t.variant == 2 || t.variant == 3 || t.variant == 17)) {
    const bool gathered = s.khw != 0 && s.ffam != 2;
    return model_estimate(mode, t.variant, s, launch_blocks(tile_for_variant(gathered ? 3 : 4), s));
  }
  return model_estimate(mode, t.variant, s, launch_blocks(t, s));
}

// The kernel chosen from the shape alone: the tile variant of the lowest
// estimate.
const Tile &choose_tile(const Shape &s, int mode) {
  int best = 3;
  double best_cost = 1e300;
  for (const Tile &t : kTiles) {
    if (t.variant == 1) continue;  // the VALU kernel: for the tests only
    // the chain kernel runs windows other than 1x1 and 3x3 as variant 6
    if (is_chain(t) && s.khw != 0 && s.khw != 1 && s.khw != 9) continue;
    if (t.variant >= 14 && t.variant <= 16 && mode == OG_MODE_EXACT) continue;  // run as 10, 13, 11
    if (t.variant == 9 && mode == OG_MODE_EXACT) continue;  // eight rows per lane: VALU-bound in exact mode
    const double e = estimate(t, s, mode);
    if (e < best_cost) {
      best_cost = e;
      best = t.variant;
    }
  }
  return tile_for_variant(best);
}


template <int KIND>
void launch(int mode, bool av, bool bv, const Tile &t, const og::Problem &p, hipStream_t s) {
  if (mode == OG_MODE_EXACT)
    launch_kind<og::kExact, KIND>(av, bv, t, p, s);
  else
    launch_kind<og::kFast, KIND>(av, bv, t, p, s);
}


const Tile &pick(const Shape &s, int mode) {
  return t_variant == 0 || t_variant == kDepthwiseVariant || t_variant == kGroupedVariant ||
                 is_split(t_variant) || is_halo(t_variant) || is_panel(t_variant)
             ? choose_tile(s, mode)
             : tile_for_variant(t_variant);
}

// The depthwise kernel with its window size compiled in where it is 3x3 or
// 5x5 (the windows of depthwise layers), read at run time otherwise.  A lane
// computes P outputs.  Measured on the MobileNetV3-large layers at batch 1
// and 8: P = 4 (or 2) pays only for 3x3 windows at stride 1, whose taps are
// contiguous loads, and only while the launch keeps at least 2048 waves;
// strided and 5x5 windows are bound by their tap loads, and fewer waves
// then only lengthen the launch.
int dw_outputs_per_lane(int64_t planes, int64_t ohw, int64_t kh, int64_t kw, int64_t sh,
                        int64_t sw) {
  if (kh != 3 || kw != 3 || sh != 1 || sw != 1) return 1;
  for (int per_lane : {4, 2})
    if (planes * ceil_div(ohw, 64 * per_lane) >= 2048) return per_lane;
  return 1;
}



void launch_rowdot(int mode, og::Problem p, bool vec, hipStream_t s) {
  if (mode == OG_MODE_EXACT)
    launch_rowdot_mode<og::kExact>(p, vec, s);
  else
    launch_rowdot_mode<og::kFast>(p, vec, s);
}

// Single-column products (n = 1, m = 1 against an N x K operand, a 1x1
// convolution of a 1x1 input): rows of more than kStreamMinK taps that can
// be read 16 bytes at a time are streamed through the chain kernel; other
// rows of up to kRowdotMaxK taps run the row-dot kernel; the rest the
// implicit product.  Measured on the squeeze-and-excitation layers and
// 4096 x 4096 matrices: the row-dot kernel halves the tile kernels' time up
// to k = 480 but its loads of 64 rows at once are bound by the texture units
// for longer rows, where the streamed form is two to three times faster.
constexpr int64_t kRowdotMaxK = 512;
constexpr int64_t kStreamMinK = 256;


void launch_chain_vt(int mode, og::Problem p, hipStream_t s) {
  if (mode == OG_MODE_EXACT)
    launch_chain_vt_mode<og::kExact>(p, s);
  else
    launch_chain_vt_mode<og::kFast>(p, s);
}

// The N x K operand can be streamed by 16-byte loads of its rows.
bool vt_ok(const float *w, int64_t ldw, int64_t k) {
  return aligned16(w) && ldw % 4 == 0 && k % 4 == 0 && k > 0 && ldw <= (int64_t(1) << 22);
}

// Blocks of the row-dot kernel address 64 rows with 32-bit byte offsets.
bool rowdot_fits(int64_t rows, int64_t ld, int64_t vstride, int64_t groups) {
  return ld <= (int64_t(1) << 22) && vstride <= (int64_t(1) << 22) &&
         ceil_div(rows, 64) * groups <= kI32Max;
}


// Tile of a product with a transposed B: the forced variant when it has a
// form for it (1..5, 17, 20), else the cheapest matrix-core tile by the
// launch model of matrix products.
const Tile &pick_nt(const Shape &sh, int mode) {
  const int v = t_variant;
  if ((v >= 1 && v <= 5) || v == 17 || v == 20) return tile_for_variant(v);
  int best = 3;
  double best_cost = 1e300;
  for (int cand : {2, 3, 4, 5, 17, 20}) {
    const double e = estimate(tile_for_variant(cand), sh, mode);
    if (e < best_cost) {
      best_cost = e;
      best = cand;
    }
  }
  return tile_for_variant(best);
}

bool grid_fits(const Tile &t, int64_t M, int64_t N, int64_t groups) {
  return ceil_div(M, t.bm) * ceil_div(N, t.bn) * groups <= kI32Max;
}

bool valid_mode(int mode) {
  return mode == OG_MODE_EXACT || mode == OG_MODE_FAST || mode == OG_MODE_FAST_MFMA;
}

// Launch time of a split-k variant: t = o + rounds * chunks * c microseconds,
// chunks = a wave's share of k in chunks of 16 taps, rounds = the launch's
// waves over cap (waves that run at once), with (cap, c, o) per variant and
// shape family (0 matrix products, 1 3x3 windows, 2 other windows), fitted
// to launches of every variant measured on the MI355X over the ResNet-50
// layers at batch 1 and 8 and a set of products (mean errors 8 to 25 %).
struct SplitCost {
  int variant, fam;
  double cap, c, o;
};
constexpr SplitCost kSplitCosts[] = {
    {21, 0, 2048, 0.4625, 3.19},
    {21, 1, 4096, 1.1671, 2.67},
    {21, 2, 4096, 1.5103, 2.33},
    {22, 0, 2048, 0.5760, 2.54},
    {22, 1, 2048, 0.7839, 3.04},
    {22, 2, 2048, 0.8099, 2.62},
    {23, 0, 2048, 0.7633, 3.19},
    {23, 1, 2048, 1.1932, 3.01},
    {23, 2, 1024, 0.8410, 2.88},
    {24, 0, 1024, 0.6900, 4.10},
    {24, 1, 1024, 0.9317, 5.80},
    {24, 2, 1024, 1.0097, 4.32},
    {25, 0, 1024, 0.4058, 3.43},
    {25, 1, 1024, 0.5304, 4.27},
    {25, 2, 1024, 0.5466, 3.73},
};
// A split-k kernel is taken only when its estimate is below this fraction
// of the fast-mode kernel's: the two estimates' errors would otherwise pick it
// where it is slower (with split-k launches of one round only; 0.85 with the
// earlier fast-mode table, 0.9 since the refitted one, whose estimates err
// less: ResNet-50 at batch 1 keeps its split-k layers).
constexpr double kSplitMargin = 0.9;

// one_round: only launches whose waves all run at once (the model's error
// grows with the rounds, and a split-k launch of several rounds was measured
// slower than the fast-mode kernels where it estimated faster).
double split_estimate(int v, const Shape &s, bool one_round) {
  const SplitTile &t = split_tile(v);
  const int fam = s.khw == 0 ? 0 : s.khw == 9 ? 1 : 2;
  for (const SplitCost &c : kSplitCosts) {
    if (c.variant != v || c.fam != fam) continue;
    const double blocks = (double)ceil_div(s.M, 16 * t.tm) * (double)ceil_div(s.N, 16 * t.tn) *
                          (double)s.groups;
    const double chunks = (double)ceil_div(ceil_div(std::max<int64_t>(s.K, 1), 16), t.ks);
    if (one_round && blocks * t.ks > c.cap) return 1e300;
    const double rounds = std::ceil(blocks * t.ks / c.cap);
    return c.o + rounds * chunks * c.c;
  }
  return 1e300;
}

// The kernel of a call in mode 2 (fast under tolerance): a split-k variant,
// or 0 for the fast-mode kernels (which meet the bound): the forced variant,
// else the lower estimate of the best fast-mode tile and the split-k tiles.
// fast_estimate < 0: no estimate of the fast path (use the split-k kernels
// only when forced).
int mode2_variant(const Shape &s, double fast_estimate) {
  if (is_split(t_variant)) return t_variant;
  if (t_variant != 0 || fast_estimate < 0) return 0;
  int best = 0;
  double best_cost = kSplitMargin * fast_estimate;
  for (const SplitTile &c : kSplitTiles) {
    const double e = split_estimate(c.variant, s, true);
    if (e < best_cost) {
      best_cost = e;
      best = c.variant;
    }
  }
  return best;
}

// The halo kernel's estimate for a 3x3 convolution whose images hold
// `tiles` tiles of 64 lanes in all (variants 26..28 and 31..33, those whose
// block fits the LDS), in exact or fast mode; the variant of the lowest.
double halo_estimate(int mode, const Shape &s, const HaloPlan &h, int64_t tiles, int *variant) {
  double best = 1e300;
  for (const int v : {26, 27, 28, 31, 32, 33}) {
    if (!halo_fits(h, v)) continue;
    const double e = model_estimate(mode, v, s, ceil_div(s.M, (int64_t)halo_block_rows(v)) * tiles * s.groups);
    if (e < best) best = e, *variant = v;
  }
  return best;
}

// The panel kernel's estimate for a product (images = 0) or a 1x1
// convolution of `images` images with ohw output pixels each (variants 29
// and 30: 16 and 32 rows per block, 64 columns); the variant of the lower.
double panel_estimate(const Shape &s, int64_t images, int *variant) {
  double best = 1e300;
  for (const auto [v, rows] : {std::pair<int, int64_t>{29, 16}, {30, 32}}) {
    const int64_t cols = images > 0 ? images * ceil_div(s.ohw, 64) : ceil_div(s.N, 64);
    const double e = model_estimate(OG_MODE_FAST, v, s, ceil_div(s.M, rows) * cols * s.groups);
    if (e < best) best = e, *variant = v;
  }
  return best;
}

// The automatic choice for a matrix product, in pieces og_gemm_f32 and
// og_gemm_choice share: the shape, the panel kernel's estimate and variant,
// the split-k variant of mode 2 (0: none), and whether the panel kernel
// beats the tile pick t (fast mode, n > 1).
Shape product_shape(int64_t m, int64_t n, int64_t k) {
  return Shape{m, n, k, 1, 0, 0, 0, 4.0 * ((double)m * k + (double)k * n + (double)m * n)};
}
double product_panel_estimate(const Shape &sh, int *panel_v) {
  *panel_v = 0;
  return ceil_div(sh.M, 16) * ceil_div(sh.N, 64) <= kI32Max ? panel_estimate(sh, 0, panel_v) : 1e300;
}
int product_split(const Shape &sh, int mode, double panel_est) {
  if (mode != OG_MODE_FAST_MFMA) return 0;
  return mode2_variant(sh, std::min(estimate(choose_tile(sh, OG_MODE_FAST), sh, OG_MODE_FAST), panel_est));
}
bool product_takes_panel(const Shape &sh, const Tile &t, double panel_est) {
  return panel_est < estimate(t, sh, OG_MODE_FAST);
}

// A split-k variant forced in exact or fast mode: refused (neither mode's
// bits can come from it).
og_status refuse_split(const char *what, int mode) {
  if (mode != OG_MODE_FAST_MFMA && is_split(t_variant))
    return fail(OG_ERR_NOT_EXACT, "%s: variant %d has no %s form (split-k kernels run only in "
                "mode 2)", what, t_variant, mode == OG_MODE_EXACT ? "exact" : "fast");
  return OG_OK;
}

}  // namespace

extern "C" {

og_status og_gemm_f32(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                      const float *B, int64_t ldb, float *C, int64_t ldc, int mode) {
  if (!valid_mode(mode))
    return fail(OG_ERR_INVALID_ARG, "og_gemm_f32: mode %d is not 0 (exact), 1 (fast) or 2 (fast "
                "under tolerance)", mode);
  if (m < 0 || n < 0 || k < 0)
    return fail(OG_ERR_INVALID_ARG, "og_gemm_f32: negative size m=%lld n=%lld k=%lld",
                (long long)m, (long long)n, (long long)k);
  if (lda < (k > 1 ? k : 1) || ldb < (n > 1 ? n : 1) || ldc < (n > 1 ? n : 1))
    return fail(OG_ERR_INVALID_ARG,
                "og_gemm_f32: leading dimension too small (lda=%lld k=%lld ldb=%lld ldc=%lld "
                "n=%lld)",
                (long long)lda, (long long)k, (long long)ldb, (long long)ldc, (long long)n);
  if (m == 0 || n == 0) return ok();
  if (C == nullptr) return fail(OG_ERR_INVALID_ARG, "og_gemm_f32: C is null");
  if (k > 0 && (A == nullptr || B == nullptr))
    return fail(OG_ERR_INVALID_ARG, "og_gemm_f32: A or B is null");
  if (m > kI32Max || n > kI32Max || k > kI32Max)
    return fail(OG_ERR_TOO_LARGE, "og_gemm_f32: a dimension exceeds 2^31-1");
  // the kernels address a tile's rows with 32-bit byte offsets
  if (lda > (int64_t(1) << 22) || ldb > (int64_t(1) << 22))
    return fail(OG_ERR_TOO_LARGE, "og_gemm_f32: lda or ldb exceeds 2^22");
  og_status st = refuse_split("og_gemm_f32", mode);
  if (st != OG_OK) return st;
  const Shape sh = product_shape(m, n, k);
  int panel_v = 0;
  const double panel_est = product_panel_estimate(sh, &panel_v);
  const int split = product_split(sh, mode, panel_est);
  if (mode == OG_MODE_FAST_MFMA && !split) mode = OG_MODE_FAST;  // the fast kernels meet the bound
  const Tile &t = pick(sh, mode);
  if (!split && !grid_fits(t, m, n, 1)) return fail(OG_ERR_TOO_LARGE, "og_gemm_f32: too many tiles");
  if (split && ceil_div(m, 16) * ceil_div(n, 16) > kI32Max)
    return fail(OG_ERR_TOO_LARGE, "og_gemm_f32: too many tiles");
  st = check_device();
  if (st != OG_OK) return st;

  og::Problem p{};
  p.A = A;
  p.lda = lda;
  p.B = B;
  p.ldb = ldb;
  p.C = C;
  p.ldc = ldc;
  p.M = (int)m;
  p.N = (int)n;
  p.K = (int)k;
  p.groups = 1;
  const bool av = aligned16(A) && lda % 4 == 0 && k % 4 == 0;
  p.a_vec = av ? 1 : 0;
  if (split) {
    launch_splitk_matrix(split, av, false, false, p, t_stream);
    return check_launch("og_gemm_f32");
  }
  // the panel kernel: forced, or chosen where its estimate is below the pick's
  if (panel_v != 0 && mode == OG_MODE_FAST && (n > 1 || is_panel(t_variant))) {
    const int pv = is_panel(t_variant)                                      ? t_variant
                   : t_variant == 0 && product_takes_panel(sh, t, panel_est) ? panel_v
                                                                            : 0;
    if (pv != 0) {
      const bool bv = aligned16(B) && ldb % 4 == 0 && n % 4 == 0;
      launch_panel(pv, og::kBMatrix, bv, av, p, t_stream);
      return check_launch("og_gemm_f32");
    }
  }
  const bool stream_col = n == 1 && k > kStreamMinK && ldb == 1 && ldc == 1 && vt_ok(A, lda, k);
  if (n == 1 && !stream_col && k <= kRowdotMaxK && t_variant == 0 && rowdot_fits(m, lda, ldb, 1)) {
    // a single column: the rows of A against the column of B
    launch_rowdot(mode, p, av, t_stream);
    return check_launch("og_gemm_f32");
  }
  if (stream_col && t_variant == 0) {
    // a long single column: B's column (contiguous) against the rows of A,
    // streamed through the chain kernel; the m outputs are C's column
    og::Problem q{};
    q.A = B;
    q.lda = k;
    q.a_vec = aligned16(B) ? 1 : 0;
    q.B = A;
    q.ldb = lda;
    q.C = C;
    q.ldc = m;
    q.M = 1;
    q.N = (int)m;
    q.K = (int)k;
    launch_chain_vt(mode, q, t_stream);
    return check_launch("og_gemm_f32");
  }
  const bool bv = aligned16(B) && ldb % 4 == 0 && n % 4 == 0;
  launch<og::kBMatrix>(mode, av, bv, t, p, t_stream);
  return check_launch("og_gemm_f32");
}

og_status og_gemm_nt_f32(int64_t m, int64_t n, int64_t k, const float *A, int64_t lda,
                         const float *B, int64_t ldb, float *C, int64_t ldc, int mode) {
  if (!valid_mode(mode))
    return fail(OG_ERR_INVALID_ARG, "og_gemm_nt_f32: mode %d is not 0 (exact), 1 (fast) or 2 "
                "(fast under tolerance)", mode);
  if (m < 0 || n < 0 || k < 0)
    return fail(OG_ERR_INVALID_ARG, "og_gemm_nt_f32: negative size m=%lld n=%lld k=%lld",
                (long long)m, (long long)n, (long long)k);
  if (lda < (k > 1 ? k : 1) || ldb < (k > 1 ? k : 1) || ldc < (n > 1 ? n : 1))
    return fail(OG_ERR_INVALID_ARG,
                "og_gemm_nt_f32: leading dimension too small (lda=%lld ldb=%lld k=%lld ldc=%lld "
                "n=%lld)",
                (long long)lda, (long long)ldb, (long long)k, (long long)ldc, (long long)n);
  if (m == 0 || n == 0) return ok();
  if (C == nullptr) return fail(OG_ERR_INVALID_ARG, "og_gemm_nt_f32: C is null");
  if (k > 0 && (A == nullptr || B == nullptr))
    return fail(OG_ERR_INVALID_ARG, "og_gemm_nt_f32: A or B is null");
  if (m > kI32Max || n > kI32Max || k > kI32Max)
    return fail(OG_ERR_TOO_LARGE, "og_gemm_nt_f32: a dimension exceeds 2^31-1");
  if (lda > (int64_t(1) << 22) || ldb > (int64_t(1) << 22))
    return fail(OG_ERR_TOO_LARGE, "og_gemm_nt_f32: lda or ldb exceeds 2^22");
  og_status st = refuse_split("og_gemm_nt_f32", mode);
  if (st != OG_OK) return st;
  const Shape sh = product_shape(m, n, k);
  const int split =
      mode == OG_MODE_FAST_MFMA
          ? mode2_variant(sh, estimate(pick_nt(sh, OG_MODE_FAST), sh, OG_MODE_FAST))
          : 0;
  if (mode == OG_MODE_FAST_MFMA && !split) mode = OG_MODE_FAST;  // the fast kernels meet the bound
  const bool single_row = m == 1 && t_variant == 0;
  const Tile &t = pick_nt(sh, mode);
  if (!split && !single_row && !grid_fits(t, m, n, 1))
    return fail(OG_ERR_TOO_LARGE, "og_gemm_nt_f32: too many tiles");
  if (split && ceil_div(m, 16) * ceil_div(n, 16) > kI32Max)
    return fail(OG_ERR_TOO_LARGE, "og_gemm_nt_f32: too many tiles");
  st = check_device();
  if (st != OG_OK) return st;
  if (split) {
    og::Problem q{};
    q.A = A;
    q.lda = lda;
    q.B = B;
    q.ldb = ldb;
    q.C = C;
    q.ldc = ldc;
    q.M = (int)m;
    q.N = (int)n;
    q.K = (int)k;
    q.groups = 1;
    const bool av = aligned16(A) && lda % 4 == 0 && k % 4 == 0;
    const bool bv = aligned16(B) && ldb % 4 == 0 && k % 4 == 0;
    q.a_vec = av ? 1 : 0;
    launch_splitk_matrix(split, av, bv, true, q, t_stream);
    return check_launch("og_gemm_nt_f32");
  }

  og::Problem p{};
  p.groups = 1;
  // few rows: up to 16, or up to 256 while 64 x 64 tiles would be fewer than
  // the chip's 256 CUs (each tile would run its whole k chain alone)
  const bool few_rows = m <= 16 || (m <= 256 && ceil_div(m, 64) * ceil_div(n, 64) < 256);
  if (few_rows && t_variant == 0 && vt_ok(B, ldb, k) && (m > 1 || k > kStreamMinK)) {
    // a few rows of A (a single row with a long k, or more) streamed against
    // the rows of B through the chain kernel, 4 rows x 16 columns per block
    og::Problem q{};
    q.A = A;
    q.lda = lda;
    q.a_vec = aligned16(A) && lda % 4 == 0 ? 1 : 0;
    q.B = B;
    q.ldb = ldb;
    q.C = C;
    q.ldc = ldc;
    q.M = (int)m;
    q.N = (int)n;
    q.K = (int)k;
    launch_chain_vt(mode, q, t_stream);
    return check_launch("og_gemm_nt_f32");
  }
  if (single_row) {
    // one row of A against the n rows of B: out[j] = sum_p B[j][p] * A[0][p]
    p.A = B;
    p.lda = ldb;
    p.B = A;
    p.ldb = 1;
    p.C = C;
    p.ldc = 1;
    p.M = (int)n;
    p.K = (int)k;
    const bool vec = aligned16(B) && ldb % 4 == 0 && k % 4 == 0;
    launch_rowdot(mode, p, vec, t_stream);
    return check_launch("og_gemm_nt_f32");
  }
  p.A = A;
  p.lda = lda;
  p.B = B;
  p.ldb = ldb;
  p.C = C;
  p.ldc = ldc;
  p.M = (int)m;
  p.N = (int)n;
  p.K = (int)k;
  const bool av = aligned16(A) && lda % 4 == 0 && k % 4 == 0;
  const bool bv = aligned16(B) && ldb % 4 == 0 && k % 4 == 0;
  p.a_vec = av ? 1 : 0;
  if (mode == OG_MODE_EXACT)
    launch_nt<og::kExact>(av, bv, t, p, t_stream);
  else
    launch_nt<og::kFast>(av, bv, t, p, t_stream);
  return check_launch("og_gemm_nt_f32");
}

int64_t og_conv2d_out_size(int64_t size, int64_t k, int64_t stride, int64_t padBefore,
                           int64_t padAfter, int64_t dil) {
  if (size < 1 || k < 1 || stride < 1 || dil < 1 || padBefore < 0 || padAfter < 0) return 0;
  const int64_t span = size + padBefore + padAfter - dil * (k - 1) - 1;
  if (span < 0) return 0;  // floor of a negative quotient plus one is < 1
  return span / stride + 1;
}

}  // extern "C"

namespace {

using namespace og::host;

// The convolution, with the epilogue (bias, activation, residual) or without
// (all null / 0).
og_status conv2d(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t G, int64_t KH,
                 int64_t KW, int64_t strideH, int64_t strideW, int64_t padTop, int64_t padLeft,
                 int64_t padBottom, int64_t padRight, int64_t dilH, int64_t dilW, const float *x,
                 const float *w, const float *bias, int act, const float *residual, float *y,
                 int mode) {
  if (!valid_mode(mode))
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32: mode %d is not 0 (exact), 1 (fast) or 2 (fast "
                "under tolerance)", mode);
  if (act != OG_ACT_NONE && act != OG_ACT_RELU)
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32_epi: activation %d is not 0 (none) or 1 (ReLU)",
                act);
  const bool epilogue = bias != nullptr || residual != nullptr || act != OG_ACT_NONE;
  if (N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || G < 1 || KH < 1 || KW < 1)
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32: sizes must be >= 1");
  if (strideH < 1 || strideW < 1 || dilH < 1 || dilW < 1)
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32: strides and dilations must be >= 1");
  if (padTop < 0 || padLeft < 0 || padBottom < 0 || padRight < 0)
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32: pads must be >= 0");
  if (Cin % G != 0 || Cout % G != 0)
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32: Cin=%lld and Cout=%lld must be multiples of "
                "G=%lld", (long long)Cin, (long long)Cout, (long long)G);
  const int64_t OH = og_conv2d_out_size(H, KH, strideH, padTop, padBottom, dilH);
  const int64_t OW = og_conv2d_out_size(W, KW, strideW, padLeft, padRight, dilW);
  if (OH < 1 || OW < 1)
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32: the window does not fit the padded input");
  if (x == nullptr || w == nullptr || y == nullptr)
    return fail(OG_ERR_INVALID_ARG, "og_conv2d_f32: null pointer");
  const int64_t cin_g = Cin / G, cout_g = Cout / G;
  const int64_t K = cin_g * KH * KW, ncols = N * OH * OW;
  // every index the kernels form in 32 bits must fit
  const int64_t dims[] = {K, ncols, Cout, H, W, OH * OW, KH * KW,
                          (H + padTop + padBottom) * strideH, (W + padLeft + padRight) * strideW,
                          KH * dilH + H, KW * dilW + W};
  for (int64_t d : dims)
    if (d > kI32Max) return fail(OG_ERR_TOO_LARGE, "og_conv2d_f32: a dimension exceeds 2^31-1");
  // the kernels address the input with 32-bit byte offsets
  if (N * Cin * H * W > (int64_t(1) << 29))
    return fail(OG_ERR_TOO_LARGE, "og_conv2d_f32: the input exceeds 2^29 elements");
  // and a tile's weight rows (K taps each, the row stride of the weights) too:
  // the same bound the matrix product puts on lda
  if (K > (int64_t(1) << 22))
    return fail(OG_ERR_TOO_LARGE, "og_conv2d_f32: Cin/G*KH*KW = %lld exceeds 2^22", (long long)K);
  const bool planes = KH == 1 && KW == 1 && strideH == 1 && strideW == 1 && padTop == 0 &&
                      padLeft == 0 && padBottom == 0 && padRight == 0;
  og_status st = refuse_split("og_conv2d_f32", mode);
  if (st != OG_OK) return st;
  Shape sh{cout_g, ncols, K, G, OH * OW, KH * KW, fast_family(KH, KW, planes, strideH, strideW),
           4.0 * ((double)N * Cin * H * W + (double)Cout * K + (double)Cout * ncols)};
  // depthwise, grouped-direct and single-column shapes keep their fast
  // kernels in mode 2 unless a split-k variant is forced
  const bool own_kernel = cin_g == 1 || (G > 1 && cin_g <= 64 && cout_g <= 8 && KH == 3 && KW == 3) ||
                          (planes && ncols == 1);
  og::Problem p{};
  p.bias = bias;
  p.res = residual;
  p.act = act;
  p.A = w;
  p.lda = K;
  p.a_gstride = cout_g * K;
  p.B = x;
  p.C = y;
  p.M = (int)cout_g;
  p.N = (int)ncols;
  p.K = (int)K;
  p.groups = (int)G;
  p.H = (int)H;
  p.W = (int)W;
  p.OW = (int)OW;
  p.OHW = (int)(OH * OW);
  p.KW = (int)KW;
  p.KH = (int)KH;
  p.HW = (int)(H * W);
  p.KHW = (int)(KH * KW);
  p.sH = (int)strideH;
  p.sW = (int)strideW;
  p.pT = (int)padTop;
  p.pL = (int)padLeft;
  p.pR = (int)padRight;
  p.dH = (int)dilH;
  p.dW = (int)dilW;
  p.x_img = Cin * H * W;
  p.x_grp = cin_g * H * W;
  p.y_img = Cout * OH * OW;
  p.y_grp = cout_g * OH * OW;
  const bool av = aligned16(w) && K % 4 == 0 && (cout_g * K) % 4 == 0;
  p.a_vec = av ? 1 : 0;
  // the halo kernel (fast mode, 3x3 windows): its staging plan and the
  // variant of the lower estimate, where it takes the shape
  HaloPlan hplan{};
  bool halo_ok = false;
  int halo_v = 0, halo_xv = 0;  // the fast and the exact variant of the lowest estimate
  double halo_est = 1e300, halo_xest = 1e300;
  if (KH == 3 && KW == 3 && !planes && !own_kernel && halo_plan(p, aligned16(x), hplan) &&
      ceil_div(cout_g, 16) * N * hplan.tiles * G <= kI32Max) {
    halo_ok = true;
    // the input floats a block stages over its k: 16 channels of hplan.rows
    // padded rows per chunk of 144 taps
    sh.halo_x = (double)K / 144.0 * 16.0 * hplan.rows * (double)(W + padLeft + padRight) * 1e-3;
    halo_est = halo_estimate(OG_MODE_FAST, sh, hplan, N * hplan.tiles, &halo_v);
    halo_xest = halo_estimate(OG_MODE_EXACT, sh, hplan, N * hplan.tiles, &halo_xv);
  }
  // the panel kernel (fast mode, 1x1 windows): its variant of the lower estimate
  int panel_v = 0;
  double panel_est = 1e300;
  if (KH == 1 && KW == 1 && !own_kernel && ceil_div(cout_g, 16) * N * ceil_div(OH * OW, 64) * G <= kI32Max)
    panel_est = panel_estimate(sh, N, &panel_v);
  const int split =
      mode == OG_MODE_FAST_MFMA
          ? mode2_variant(sh, own_kernel ? -1.0
                                         : std::min({estimate(choose_tile(sh, OG_MODE_FAST), sh, OG_MODE_FAST),
                                                     halo_est, panel_est}))
          : 0;
  if (mode == OG_MODE_FAST_MFMA && !split) mode = OG_MODE_FAST;  // the fast kernels meet the bound
  const Tile &t = pick(sh, mode);
  if (!split && !grid_fits(t, cout_g, ncols, G))
    return fail(OG_ERR_TOO_LARGE, "og_conv2d_f32: too many tiles");
  if (split && ceil_div(cout_g, 16) * ceil_div(ncols, 16) * G > kI32Max)
    return fail(OG_ERR_TOO_LARGE, "og_conv2d_f32: too many tiles");
  st = check_device();
  if (st != OG_OK) return st;

  if (cin_g == 1 && (t_variant == 0 || t_variant == kDepthwiseVariant)) {
    // depthwise: one wave per 64 * per_lane output pixels of an (image, output channel) plane
    const int per_lane = dw_outputs_per_lane(N * Cout, OH * OW, KH, KW, strideH, strideW);
    const int64_t per_plane = ceil_div(OH * OW, 64 * per_lane), nplanes = N * Cout;
    if (per_plane * nplanes > kI32Max - 3)
      return fail(OG_ERR_TOO_LARGE, "og_conv2d_f32: too many output planes");
    if (by_mode_epi<DwBand>(mode, epilogue, p, nplanes, OH, OW, t_stream))
      return check_launch("og_conv2d_f32");
    p.tiles_m = (int)per_plane;
    p.tiles_n = (int)nplanes;
    by_mode_epi<Dw>(mode, epilogue, p, per_lane, t_stream);
    return check_launch("og_conv2d_f32");
  }
  if (G > 1 && cin_g >= 2 && cin_g <= 64 && cout_g <= 8 && KH == 3 && KW == 3 &&
      (t_variant == 0 || t_variant == kGroupedVariant) &&
      ceil_div(OH * OW, 64) * N * G <= kI32Max - 3) {
    // grouped, few output channels per group: one wave per 64 output pixels of
    // an (image, group), all of the group's output channels per lane
    p.tiles_m = (int)ceil_div(OH * OW, 64);
    p.tiles_n = (int)(N * G);
    by_mode_epi<Grouped>(mode, epilogue, p, t_stream);
    return check_launch("og_conv2d_f32");
  }
  if (split) {
    launch_splitk_conv(split, av, planes, p, t_stream);
    return check_launch("og_conv2d_f32");
  }
  // the halo kernel: forced, or chosen where its estimate is below the pick's
  if (halo_ok && (mode == OG_MODE_FAST || mode == OG_MODE_EXACT)) {
    const int best_v = mode == OG_MODE_EXACT ? halo_xv : halo_v;
    const double best_est = mode == OG_MODE_EXACT ? halo_xest : halo_est;
    // (a forced variant whose block does not fit the LDS runs as 0 does)
    const bool forced = is_halo(t_variant) && halo_fits(hplan, t_variant);
    const bool automatic = t_variant == 0 || (is_halo(t_variant) && !forced);
    const int hv = forced ? t_variant
                   : automatic && best_v != 0 && best_est < estimate(t, sh, mode) ? best_v
                                                                                  : 0;
    if (hv != 0) {
      launch_halo_conv(hv, mode, p, hplan, t_stream);
      return check_launch("og_conv2d_f32");
    }
  }
  // the panel kernel: forced, or chosen where its estimate is below the pick's
  if (panel_v != 0 && mode == OG_MODE_FAST) {
    const int pv = is_panel(t_variant) ? t_variant
                   : t_variant == 0 && panel_est < estimate(t, sh, mode) ? panel_v
                                                                         : 0;
    if (pv != 0) {
      const bool bv = planes && aligned16(x) && (H * W) % 4 == 0 && p.x_img % 4 == 0 && p.x_grp % 4 == 0;
      launch_panel(pv, planes ? og::kBPlanes : og::kBGather, bv, av, p, t_stream);
      return check_launch("og_conv2d_f32");
    }
  }
  // (the streamed form's outputs are its columns, not its rows: no epilogue there)
  const bool stream_se = planes && ncols == 1 && G == 1 && K > kStreamMinK && vt_ok(w, K, K) &&
                         !epilogue;
  if (planes && ncols == 1 && !stream_se && K <= kRowdotMaxK && t_variant == 0 &&
      rowdot_fits(cout_g, K, 1, G)) {
    // a 1x1 convolution of one 1x1 input: per group, the weight rows against
    // the group's input channels
    p.ldb = 1;
    p.ldc = 1;
    launch_rowdot(mode, p, av, t_stream);
    return check_launch("og_conv2d_f32");
  }
  if (stream_se && t_variant == 0) {
    // a long 1x1 convolution of one 1x1 input: the input channels against
    // the weight rows, streamed through the chain kernel
    og::Problem q{};
    q.A = x;
    q.lda = K;
    q.a_vec = aligned16(x) ? 1 : 0;
    q.B = w;
    q.ldb = K;
    q.C = y;
    q.ldc = Cout;
    q.M = 1;
    q.N = (int)Cout;
    q.K = (int)K;
    launch_chain_vt(mode, q, t_stream);
    return check_launch("og_conv2d_f32");
  }
  if (planes)
    launch<og::kBPlanes>(mode, av, false, t, p, t_stream);
  else
    launch<og::kBGather>(mode, av, false, t, p, t_stream);
  return check_launch("og_conv2d_f32");
}

}  // namespace

extern "C" {

og_status og_conv2d_f32_ex(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                           int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                           int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                           int64_t dilH, int64_t dilW, const float *x, const float *w, float *y,
                           int mode) {
  return conv2d(N, Cin, H, W, Cout, G, KH, KW, strideH, strideW, padTop, padLeft, padBottom,
                padRight, dilH, dilW, x, w, nullptr, OG_ACT_NONE, nullptr, y, mode);
}

og_status og_conv2d_f32_epi(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                            int64_t G, int64_t KH, int64_t KW, int64_t strideH, int64_t strideW,
                            int64_t padTop, int64_t padLeft, int64_t padBottom, int64_t padRight,
                            int64_t dilH, int64_t dilW, const float *x, const float *w,
                            const float *bias, int act, const float *residual, float *y,
                            int mode) {
  return conv2d(N, Cin, H, W, Cout, G, KH, KW, strideH, strideW, padTop, padLeft, padBottom,
                padRight, dilH, dilW, x, w, bias, act, residual, y, mode);
}

og_status og_conv2d_f32(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout, int64_t G,
                        int64_t KH, int64_t KW, int64_t stride, int64_t pad, int64_t dil,
                        const float *x, const float *w, float *y, int mode) {
  return og_conv2d_f32_ex(N, Cin, H, W, Cout, G, KH, KW, stride, stride, pad, pad, pad, pad, dil,
                          dil, x, w, y, mode);
}

og_status og_set_stream(void *hip_stream) {
  t_stream = static_cast<hipStream_t>(hip_stream);
  return ok();
}

void *og_get_stream(void) { return t_stream; }

og_status og_set_variant(int variant) {
  if (variant < 0 || variant > kLastHaloDppVariant)
    return fail(OG_ERR_INVALID_ARG, "og_set_variant: %d is not in 0..%d", variant,
                kLastHaloDppVariant);
  t_variant = variant;
  return ok();
}

int og_get_variant(void) { return t_variant; }

int og_gemm_choice(int64_t m, int64_t n, int64_t k, int mode) {
  if (!valid_mode(mode))
    return fail(OG_ERR_INVALID_ARG, "og_gemm_choice: mode %d is not 0, 1 or 2", mode);
  if (m < 1 || n < 2 || k < 1)
    return fail(OG_ERR_INVALID_ARG, "og_gemm_choice: needs m >= 1, n >= 2, k >= 1 (m=%lld n=%lld k=%lld)",
                (long long)m, (long long)n, (long long)k);
  if (m > kI32Max || n > kI32Max || k > kI32Max)
    return fail(OG_ERR_TOO_LARGE, "og_gemm_choice: a dimension exceeds 2^31-1");
  const Shape sh = product_shape(m, n, k);
  int panel_v = 0;
  const double panel_est = product_panel_estimate(sh, &panel_v);
  const int split = product_split(sh, mode, panel_est);
  if (split) {
    ok();
    return split;
  }
  if (mode == OG_MODE_FAST_MFMA) mode = OG_MODE_FAST;
  const Tile &t = choose_tile(sh, mode);
  ok();
  return panel_v != 0 && mode == OG_MODE_FAST && product_takes_panel(sh, t, panel_est) ? panel_v : t.variant;
}

const char *og_last_error(void) { return t_error.c_str(); }

const char *og_version(void) { return "0.1.0"; }

}  // extern "C"
