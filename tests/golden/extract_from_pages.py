"""Write the worked examples printed on the operator pages as JSON fixtures.

Reads the extracted text of the pages (a markdown file with each page under
its address; its path is the one argument) and writes, next to this script:

  affine_grid_examples.json  -- the four worked examples of the AffineGrid page
  grid_sample_examples.json  -- the eighteen worked examples of the
                                "GridSample - version 20" page
  resize_examples.json       -- the Resize (version 18) examples, all but
                                the antialias and tf_crop_and_resize ones
  deform_conv_examples.json  -- the four DeformConv (version 22) examples

Only numbers the pages print are stored (inputs, attributes, printed outputs),
each with the page title and example name it came from.  Nothing here computes
an expected value.  Run:  python tests/golden/extract_from_pages.py PAGES_TEXT
"""

from __future__ import annotations

import json
import os
import re
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

NUM = re.compile(r"[-+]?(?:\d+\.?\d*|\.\d+)(?:[eE][-+]?\d+)?")


def numbers(text: str):
    return [float(t) for t in NUM.findall(text)]


def prod(shape):
    p = 1
    for s in shape:
        p *= s
    return p


def parse_shape(s: str):
    return [int(v) for v in re.findall(r"\d+", s)]


def page_text(lines, first_marker, last_marker):
    start = next(i for i, l in enumerate(lines) if first_marker in l)
    end = next(i for i, l in enumerate(lines) if i > start and last_marker in l)
    return lines[start:end]


def tensor_after(block: str, label: str):
    """Shape and values of the tensor printed after 'label: shape=(...)'."""
    m = re.search(re.escape(label) + r": shape=\(([^)]*)\), dtype=(\w+)", block)
    if not m:
        raise ValueError("no tensor %r" % label)
    shape = parse_shape(m.group(1))
    rest = block[m.end():]
    # the values are the first bracketed block after the header
    i = rest.index("[")
    depth = 0
    for j in range(i, len(rest)):
        if rest[j] == "[":
            depth += 1
        elif rest[j] == "]":
            depth -= 1
            if depth == 0:
                break
    vals = numbers(rest[i:j + 1])
    if len(vals) != prod(shape if shape else [1]):
        raise ValueError("%s: %d values for shape %s" % (label, len(vals), shape))
    return shape, m.group(2), vals


def affine_grid_examples(lines):
    text = page_text(lines, "page 1 of 5", "page 2 of 5")
    names = [l.strip() for l in text if re.fullmatch(r"test_affine_grid_\w+", l.strip())]
    joined = "\n".join(text)
    out = []
    for k, name in enumerate(names):
        start = joined.index("\n" + name + "\n")
        end = joined.index("\n" + names[k + 1] + "\n") if k + 1 < len(names) else len(joined)
        block = joined[start:end]
        ac = int(re.search(r"align_corners = (\d)", block).group(1))
        th_shape, th_dtype, th = tensor_after(block, "theta")
        sz_shape, _, sz = tensor_after(block, "size")
        g_shape, g_dtype, g = tensor_after(block, "grid")
        out.append({
            "name": name,
            "citation": "AffineGrid page (onnx-light, since version 20), Examples: " + name,
            "align_corners": ac,
            "theta_shape": th_shape, "theta": th,
            "size": [int(v) for v in sz],
            "grid_shape": g_shape, "grid_dtype": g_dtype, "grid": g,
        })
    return out


def grid_sample_examples(lines):
    text = page_text(lines, "page 3 of 5", "Differences with previous version")
    joined = "\n".join(text)
    heads = [(m.start(), m.group(1)) for m in re.finditer(r"\*\*(test_gridsample\w*)\*\*", joined)]
    out = []
    for k, (pos, name) in enumerate(heads):
        end = heads[k + 1][0] if k + 1 < len(heads) else len(joined)
        block = joined[pos:end]
        attrs = block[:block.index("Inputs:")]
        mode = re.search(r'mode = "(\w+)"', re.sub(r"padding_mode", "", attrs))
        pad = re.search(r'padding_mode = "(\w+)"', attrs)
        ac = re.search(r"align_corners = (\d)", attrs)
        x_shape, x_dtype, x = tensor_after(block, "X")
        g_shape, g_dtype, g = tensor_after(block, "Grid")
        y_shape, y_dtype, y = tensor_after(block, "Y")
        out.append({
            "name": name,
            "citation": "GridSample - version 20 page (onnx-light), Examples: " + name,
            "mode": mode.group(1) if mode else None,
            "padding_mode": pad.group(1) if pad else None,
            "align_corners": int(ac.group(1)) if ac else None,
            "X_shape": x_shape, "X_dtype": x_dtype, "X": x,
            "grid_shape": g_shape, "grid_dtype": g_dtype, "grid": g,
            "Y_shape": y_shape, "Y_dtype": y_dtype, "Y": y,
        })
    return out


# Resize examples: every one on the page except the antialias and
# tf_crop_and_resize ones (other filters and a region of interest, outside
# what the library implements).
RESIZE_SKIP = ("antialias", "tf_crop_and_resize")


def bracket_block(s: str, i: int):
    depth = 0
    for j in range(i, len(s)):
        if s[j] == "[":
            depth += 1
        elif s[j] == "]":
            depth -= 1
            if depth == 0:
                return s[i:j + 1], j + 1
    raise ValueError("unbalanced brackets")


def nested_shape(txt: str):
    """Shape of a printed nested list (rows may wrap)."""
    depth = txt[:txt.index(next(c for c in txt if c.isdigit() or c == "-"))].count("[")
    rows = re.findall(r"\[([^\[\]]+)\]", txt)
    return [1] * (depth - 2) + [len(rows), len(numbers(rows[0]))]


def resize_examples(lines):
    # The Resize version 18 section is collapsed onto one very long line.
    text = page_text(lines, "page 2 of 5", "page 3 of 5")
    line = max(text, key=len)
    heads = [(m.start(), m.group(1)) for m in re.finditer(r"\*\*_(resize_\w+)\*\*", line)]
    out = []
    for k, (head, short) in enumerate(heads):
        name = "test_" + short
        if any(tag in name for tag in RESIZE_SKIP):
            continue
        end = heads[k + 1][0] if k + 1 < len(heads) else len(line)
        block = line[head:end]
        # Examples are keyed by their heading; the listing's own test name is
        # kept too (on the page the not_smaller upsample listing repeats the
        # not_larger name).
        listed = re.findall(r'name="(test_resize_\w+)"', block)
        if len(listed) != 1:
            raise ValueError("example %s not delimited as expected" % name)
        node = block[block.index("make_node("):block.index("data = np.array(")]
        attr = {}
        for key in ("mode", "coordinate_transformation_mode", "nearest_mode"):
            m = re.search(r'\b%s="(\w+)"' % key, node)
            attr[key] = m.group(1) if m else None
        m = re.search(r"cubic_coeff_a=(-?[\d.]+)", node)
        attr["cubic_coeff_a"] = float(m.group(1)) if m else None
        attr["exclude_outside"] = 1 if re.search(r"exclude_outside=(True|1)", node) else 0
        m = re.search(r"axes = \[([^\]]*)\]", block)
        attr["axes"] = [int(v) for v in numbers(m.group(1))] if m else None
        m = re.search(r'keep_aspect_ratio_policy = "(\w+)"', block)
        attr["keep_aspect_ratio_policy"] = m.group(1) if m else None
        d0 = block.index("data = np.array(") + len("data = np.array(")
        data_txt, _ = bracket_block(block, block.index("[", d0))
        scales = sizes = None
        m = re.search(r"scales = np\.array\(\[([^\]]*)\]", block)
        if m:
            scales = numbers(m.group(1))
        m = re.search(r"sizes = np\.array\(\[([^\]]*)\]", block)
        if m:
            sizes = [int(v) for v in numbers(m.group(1))]
        # the printed expected output is the commented block before "output ="
        c0 = block.index("# [[[[")
        c1 = block.index("output =", c0)
        printed = block[c0:c1].replace("#", " ")
        exp_txt, _ = bracket_block(printed, printed.index("["))
        # the aspect-ratio examples also state the output extents in words
        m = re.search(r"# Results in (\d+)x(\d+)", block)
        attr["results_in"] = [int(m.group(1)), int(m.group(2))] if m else None
        out.append({
            "name": name,
            "citation": "Resize page (mlprodict, version 18), Examples: " + name,
            "listing_name": listed[0],
            **attr,
            "data_shape": nested_shape(data_txt), "data": numbers(data_txt),
            "scales": scales, "sizes": sizes,
            "expected_shape": nested_shape(exp_txt), "expected": numbers(exp_txt),
        })
    return out


def bracket_values(block: str, label: str):
    """Shape and printed text of the tensor after 'label: shape=(...)'."""
    m = re.search(re.escape(label) + r": shape=\(([^)]*)\), dtype=(\w+)", block)
    if not m:
        return None
    rest = block[m.end():]
    txt, _ = bracket_block(rest, rest.index("["))
    return parse_shape(m.group(1)), m.group(2), txt


def deform_conv_examples(lines):
    # The DeformConv page is collapsed onto one long line; one example's
    # offset tensor is printed with numpy's summarisation ("...") over its
    # channel axis: the channels it prints are kept, the elided ones are
    # listed under "elided_channels" and stored as zeros (a reading: the
    # printed output is reproduced with them zero).
    text = page_text(lines, "page 4 of 5", "page 5 of 5")
    line = max(text, key=len)
    heads = [(m.start(), m.group(1)) for m in re.finditer(r"\*\*(test_cc_\w+)\*\*", line)]
    out = []
    for k, (pos, name) in enumerate(heads):
        end = heads[k + 1][0] if k + 1 < len(heads) else line.index("Differences with previous")
        block = line[pos:end]
        attrs = block[block.index("Attributes:"):block.index("Inputs:")]
        ex = {"name": name,
              "citation": "DeformConv page (onnx-light, since version 22), Examples: " + name}
        for key in ("kernel_shape", "pads", "strides", "dilations"):
            m = re.search(key + r" = \[([^\]]*)\]", attrs)
            ex[key] = [int(v) for v in numbers(m.group(1))] if m else None
        for key in ("offset_group", "group"):
            m = re.search(r"\b" + key + r" = (\d+)", attrs)
            ex[key] = int(m.group(1)) if m else None
        for label in ("X", "W", "offset", "B", "mask", "Y"):
            got = bracket_values(block, label)
            if got is None:
                ex[label] = None
                continue
            shape, dtype, txt = got
            elided = []
            if "..." in txt:
                # channel blocks of the (1, C, h, w) tensor around the ellipsis
                # strip the batch bracket and the n = 0 bracket
                inner = txt[txt.index("[") + 1:txt.rindex("]")]
                nblock, _ = bracket_block(inner, inner.index("["))
                inner = nblock[1:-1]
                parts = []
                i = 0
                while i < len(inner):
                    if inner[i] == "[":
                        b, i = bracket_block(inner, i)
                        parts.append(b)
                    elif inner.startswith("...", i):
                        parts.append("...")
                        i += 3
                    else:
                        i += 1
                head = parts[:parts.index("...")]
                tail = parts[parts.index("...") + 1:]
                per = prod(shape[2:])
                elided = list(range(len(head), shape[1] - len(tail)))
                vals = []
                for b in head:
                    vals += numbers(b)
                vals += [0.0] * (per * len(elided))
                for b in tail:
                    vals += numbers(b)
            else:
                vals = numbers(txt)
            if len(vals) != prod(shape):
                raise ValueError("%s %s: %d values for %s" % (name, label, len(vals), shape))
            ex[label] = {"shape": shape, "dtype": dtype, "values": vals}
            if elided:
                ex[label]["elided_channels"] = elided
        out.append(ex)
    return out


def main():
    if len(sys.argv) != 2 or not os.path.exists(sys.argv[1]):
        sys.exit("usage: extract_from_pages.py PAGES_TEXT (the extracted page text)")
    with open(sys.argv[1], encoding="utf-8") as f:
        lines = f.read().split("\n")
    for fname, items in (("affine_grid_examples.json", affine_grid_examples(lines)),
                         ("grid_sample_examples.json", grid_sample_examples(lines)),
                         ("resize_examples.json", resize_examples(lines)),
                         ("deform_conv_examples.json", deform_conv_examples(lines))):
        with open(os.path.join(HERE, fname), "w") as f:
            json.dump(items, f, indent=0)
            f.write("\n")
        print("%s: %d examples" % (fname, len(items)))


if __name__ == "__main__":
    main()
